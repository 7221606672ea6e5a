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
// exact. Diagonal sub-chunk blocks (factors up to e^{75}) run on the fp32
// MFMA. fp32 inputs run every product on the fp32 MFMA.
#include "kda_common.h"
#include "kda_internal.h"

#include <atomic>

namespace kda {

constexpr int KP = kHeadDim + 4;   // LDS row pitch (floats) of [C][128] tiles

size_t record_bytes(int chunk, bool precise, int D) {
    if (D == 64) return (chunk == 64 && !precise) ? Record<64, false, 64>::BYTES : 0;
    if (D == 256) return (chunk == 64 && !precise) ? Record<64, false, 256>::BYTES : 0;
    if (D != 128) return 0;
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
    static __device__ __forceinline__ void store_half(void *p, const float (&x)[8]) {   // x[0..3]
        typedef _Float16 half4 __attribute__((ext_vector_type(4)));
        *(half4 *)p = half4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
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
    static __device__ __forceinline__ void store_half(void *p, const float (&x)[8]) {   // x[0..3]
        *(f32x4 *)p = f32x4{x[0], x[1], x[2], x[3]};
    }
    static __device__ __forceinline__ f32x4 mma(const T &a, const T &b, f32x4 c) {
        return mfma_f32x8(a.v, b.v, c);
    }
    static constexpr int BYTES = 32;
};

__device__ __forceinline__ float inv_pow2(float s) {   // exact 1/s for s = 2^e
    return __uint_as_float((uint32_t)(254 - (int)((__float_as_uint(s) >> 23) & 0xFF)) << 23);
}

// 16x16x16 fp32 product on the fp32 MFMA (four 16x16x4 steps). `a` holds row
// lr of the left factor at columns 4 lg .. 4 lg + 3, `b` holds rows
// 4 lg .. 4 lg + 3 of the right factor at column lr: exactly what an
// accumulator tile holds, so a product can feed the next one as its right
// factor without leaving registers (lr = lane % 16, lg = lane / 16).
__device__ __forceinline__ f32x4 mm16(const f32x4 &a, const f32x4 &b, f32x4 acc) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk], b[kk], acc, 0, 0, 0);
    return acc;
}
// Left-factor operand of a 16x16 LDS block (row stride ld floats, 16-byte aligned rows).
__device__ __forceinline__ f32x4 lds_left16(const float *blk, int ld, int lr, int lg) {
    return *(const f32x4 *)(blk + lr * ld + 4 * lg);
}
// Right-factor operand (accumulator layout) of a 16x16 LDS block.
__device__ __forceinline__ f32x4 lds_right16(const float *blk, int ld, int lr, int lg) {
    return f32x4{blk[(4 * lg) * ld + lr], blk[(4 * lg + 1) * ld + lr], blk[(4 * lg + 2) * ld + lr],
                 blk[(4 * lg + 3) * ld + lr]};
}
__device__ __forceinline__ void lds_store16(float *blk, int ld, const f32x4 &d, int lr, int lg) {
#pragma unroll
    for (int i = 0; i < 4; ++i) blk[(4 * lg + i) * ld + lr] = d[i];
}

// Locate chunk `slot` of the packed batch: returns false for an unused slot.
template <int C>
__device__ __forceinline__ bool locate_slot(const int64_t *cu_ptr, int N, int64_t slot,
                                            int &n, int64_t &t0, int &L) {
    // the offsets are read-only for the whole launch: the constant address
    // space lets these wave-uniform reads go through the scalar cache
    const __attribute__((address_space(4))) int64_t *cu =
        (const __attribute__((address_space(4))) int64_t *)cu_ptr;
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
// Intra-chunk kernel: persistent workgroups (8 waves) over the (chunk slot,
// head) tiles; tile i is record i of the workspace (slot * H + head).
//
// LDS holds three [C][128] fp32 tiles rewritten in place as the phases go:
// sQ = qh -> qh*P;  sK = kh -> kh*P;  sP = alpha -> P -> kh/P -> v (scaled),
// with P_t the block-local prefix product of alpha. Every operand of A and M is
// one of those rows times at most one per-(block, channel) factor. Once the
// W/Ub operands are in registers the three tiles are free: the next tile's raw
// inputs are copied there (global->LDS, no registers) during the inverse and
// the W/Ub products (bf16 inputs; fp32 inputs do not fit and are read directly).
// =============================================================================
constexpr int kIntraWaves = 8;

template <int C, typename Tin>
struct RawLayout {                    // raw inputs of one tile inside the three LDS tiles
    static constexpr size_t Q = 0;
    static constexpr size_t K = Q + (size_t)C * kHeadDim * sizeof(Tin);
    static constexpr size_t V = K + (size_t)C * kHeadDim * sizeof(Tin);
    static constexpr size_t G = V + (size_t)C * kHeadDim * sizeof(Tin);
    static constexpr size_t B = G + (size_t)C * kHeadDim * 4;
    static constexpr size_t DT = B + (size_t)C * 4;              // dt_bias row of the head
    static constexpr size_t BYTES = DT + (size_t)kHeadDim * 4;
    static constexpr int NQ16 = (int)((size_t)C * kHeadDim * sizeof(Tin) / 16);  // 16-B pieces
    static constexpr int NG16 = C * kHeadDim * 4 / 16;
    static constexpr int PER = (3 * NQ16 + NG16 + 64 * kIntraWaves - 1) / (64 * kIntraWaves);
    static constexpr bool FITS = BYTES <= (size_t)3 * C * (kHeadDim + 4) * 4;
};

// Start copying one tile's raw inputs into LDS (layout RawLayout): 16-byte
// pieces of q, k, v (row-major [C][128]) and g, plus beta and the head's
// dt_bias, as asynchronous
// global->LDS copies; piece idx = tid + NT * i lands at byte 16 idx, so each
// wave fills contiguous 1 KiB blocks. Rows past the chunk end copy the chunk's
// last row (in bounds for a valid tile) and are masked where used. The caller
// waits (wait_vmem + lds_barrier) before reading.
template <int C, typename Tin, int PART = 2>
__device__ __forceinline__ void stage_raw(const PrefillArgs &p, int h, int64_t t0, int L, int tid,
                                          unsigned char *lds) {
    using RL = RawLayout<C, Tin>;
    constexpr int NT = 64 * kIntraWaves;
    constexpr uint32_t RB = kHeadDim * (uint32_t)sizeof(Tin);   // bytes per q/k/v row
    constexpr int PPR = (int)RB / 16;                            // pieces per q/k/v row
    static_assert(RL::NQ16 % 64 == 0 && RL::NG16 % 64 == 0, "a wave's pieces stay in one array");
    // PART 0: q and k; PART 1: v, g, beta and dt_bias; PART 2: everything
    constexpr int P0 = PART == 1 ? 2 * RL::NQ16 : 0;
    constexpr int P1 = PART == 0 ? 2 * RL::NQ16 : 3 * RL::NQ16 + RL::NG16;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    // resources over rows t0 .. t0 + L - 1 of head h (token stride H rows; q and k
    // of its q/k head h / (H / Hk), token stride Hk rows)
    const size_t row0 = (size_t)t0 * p.H + h;
    const size_t rowk0 = (size_t)t0 * p.Hk + h / (p.H / p.Hk);
    const uint32_t hq = (uint32_t)p.H * RB, hg = (uint32_t)p.H * 512u;
    const uint32_t hk = (uint32_t)p.Hk * RB;
    const uint32_t span = (uint32_t)(L - 1);
    const i32x4 rq = make_rsrc((const unsigned char *)p.q + rowk0 * RB, span * hk + RB);
    const i32x4 rk = make_rsrc((const unsigned char *)p.k + rowk0 * RB, span * hk + RB);
    const i32x4 rv = make_rsrc((const unsigned char *)p.v + row0 * RB, span * hq + RB);
    const i32x4 rg = make_rsrc(p.g + row0 * kHeadDim, span * hg + 512u);
#pragma unroll
    for (int i = 0; i < (P1 - P0 + NT - 1) / NT; ++i) {
        const int wbase = P0 + 64 * wave + NT * i;              // first piece of this wave
        if (wbase >= P1) break;                                 // whole wave past the end
        const uint32_t idx = (uint32_t)(wbase + lane);
        if (wbase < 3 * RL::NQ16) {
            const int arr = wbase / RL::NQ16;
            const uint32_t w = idx % (uint32_t)RL::NQ16;
            const uint32_t t = min(w / (uint32_t)PPR, span);
            const uint32_t off = t * (arr == 2 ? hq : hk) + (w % (uint32_t)PPR) * 16u;
            copy16_to_lds(arr == 0 ? rq : arr == 1 ? rk : rv, off, 0, lds + (size_t)wbase * 16);
        } else {
            const uint32_t w = idx - 3u * RL::NQ16;
            const uint32_t t = min(w / 32u, span);
            copy16_to_lds(rg, t * hg + (w % 32u) * 16u, 0, lds + (size_t)wbase * 16);
        }
    }
    if constexpr (PART != 0) {
        if (wave == 0) {                                         // beta, one float per row
            const i32x4 rb = make_rsrc(p.beta_raw + row0, span * (uint32_t)p.H * 4u + 4u);
            const uint32_t t = min((uint32_t)tid, span);
            if (tid < C) copy4_to_lds(rb, t * (uint32_t)p.H * 4u, 0, lds + RL::B);
        } else if (wave == 1) {                                  // dt_bias[h], 512 bytes
            const i32x4 rd = make_rsrc(p.dt_bias + (size_t)h * kHeadDim, 512u);
            if (lane < 32) copy16_to_lds(rd, 16u * (uint32_t)lane, 0, lds + RL::DT);
        }
    }
}

// 8 entries of a row of T = X diag(beta): X from LDS scaled by beta per column.
__device__ __forceinline__ void load_T_row(const float *x, const float *beta, float (&t)[8]) {
    float b[8];
    load8(x, t);
    load8(beta, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] *= b[e];
}

template <int C, typename Tin, bool PRECISE>
__global__ __launch_bounds__(64 * kIntraWaves) void intra_kernel(PrefillArgs p, int64_t ntiles)
{
    using G = ChunkGeom<C>;
    using R = Record<C, PRECISE>;
    using F = Frag<PRECISE>;
    using RL = RawLayout<C, Tin>;
    constexpr bool PF = RL::FITS;              // park the next tile's inputs in LDS
    constexpr int RG = C / 4, RIT = (RG + kIntraWaves - 1) / kIntraWaves;
    constexpr int NB = G::NB, CS = G::CS, NW = kIntraWaves, NT = 64 * NW;
    constexpr int AP = C + 4;
    constexpr int NPO = NB * (NB - 1) / 2 + 1;   // off-diagonal block pairs (+1: never empty)

    __shared__ __align__(16) float sBig[3][C][KP];
    float (*sQ)[KP] = sBig[0];
    float (*sK)[KP] = sBig[1];
    float (*sP)[KP] = sBig[2];
    unsigned char *sRaw = (unsigned char *)&sBig[0][0][0];
    __shared__ __align__(16) float sA[C][AP];   // A, strictly lower, beta-scaled
    __shared__ __align__(16) float sT[C][AP];   // T
    __shared__ __align__(16) float sA0[NB][kHeadDim];  // alpha of each block's first row
    __shared__ __align__(16) float sPe[NB][kHeadDim];  // P at each block's last row
    __shared__ __align__(16) float sQF[NB][kHeadDim];  // prod alpha over rows 0 .. 16b
    __shared__ __align__(16) float sKF[NB][kHeadDim];  // prod alpha over rows 16b+1 .. C-1
    __shared__ __align__(16) float sEF[NPO][kHeadDim]; // prod alpha over rows 16b+1 .. 16a
    __shared__ __align__(16) float sBeta[C];
    __shared__ __align__(16) float sX[NB][16][20];   // per diagonal block: inverse scratch
    __shared__ float sVmax[NW];
    __shared__ int sJob;                                // next unclaimed light job of phase 2

    const int H = p.H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lr = lane & 15, lg = lane >> 4;
    const int c8 = 8 * lr;
    const float lb2 = p.lower_bound * kLog2e;

    int64_t ti = blockIdx.x;
    int n = 0, L = 0;
    int64_t t0 = 0;
    bool valid = ti < ntiles && locate_slot<C>(p.cu_seqlens, p.N, ti / H, n, t0, L);
    if constexpr (PF) {
        if (valid) stage_raw<C, Tin>(p, (int)(ti % H), t0, L, tid, sRaw);
        wait_vmem();
        lds_barrier();
    }

    // W and Ub fragments of the previous tile, stored during the next tile's
    // phase 1 (VALU-bound, the memory queue idle) rather than at the end of
    // their own tile, where they would queue behind the input copies
    typedef std::conditional_t<PRECISE, f32x4, half4_t> UbT;
    typename F::T pend_w[2];
    UbT pend_u[NB];
    unsigned char *pend_rec = nullptr;
    auto flush = [&]() {
        if (pend_rec) {
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const int tb = 2 * (wave >> 2) + q2;
                if (tb < NB)
                    *(typename F::T *)(pend_rec + R::W_OFF + ((size_t)(tb * 4 + (wave & 3)) * 64 + lane) * F::BYTES) =
                        pend_w[q2];
            }
#pragma unroll
            for (int tb = 0; tb < NB; ++tb)
                *(UbT *)(pend_rec + R::UB_OFF + ((size_t)(wave * NB + tb) * 64 + lane) * 4 * R::UB_ELT) = pend_u[tb];
            pend_rec = nullptr;
        }
    };

    for (; ti < ntiles; ) {
        const int64_t next = ti + gridDim.x;
        if (!valid) {                            // unused slot: nothing to compute
            ti = next;
            valid = ti < ntiles && locate_slot<C>(p.cu_seqlens, p.N, ti / H, n, t0, L);
            if constexpr (PF) {
                if (valid) stage_raw<C, Tin>(p, (int)(ti % H), t0, L, tid, sRaw);
                wait_vmem();
                lds_barrier();
            }
            continue;
        }
        const int h = (int)(ti % H);
        const int Lc = L;
        const int64_t t0c = t0;
        unsigned char *rec = p.ws + (size_t)ti * R::BYTES;
        // where the next tile lies, resolved now while nothing is in flight
        int n_nx = 0, L_nx = 0;
        int64_t t0_nx = 0;
        const bool valid_nx = next < ntiles && locate_slot<C>(p.cu_seqlens, p.N, next / H, n_nx, t0_nx, L_nx);

        flush();
        // ---- phase 1: a DPP row of 16 lanes per token, 8 channels per lane -------
        // gate: sigmoid(a (g + db)) = 1 / (1 + 2^(ga g + gb)), ga = -a log2e, gb = ga db;
        // 2^x overflows to inf for very negative arguments and 1/inf = 0, so this
        // form is exact at both ends.
        const float alog = *(const __attribute__((address_space(4))) float *)(p.A_log + h);
        const float ga = -fast_exp2(alog * kLog2e) * kLog2e;
        float gb[8];
        if constexpr (PF) load8((const float *)(sRaw + RL::DT) + c8, gb);   // staged with the tile
        else load8(p.dt_bias + h * kHeadDim + c8, gb);
#pragma unroll
        for (int e = 0; e < 8; ++e) gb[e] *= ga;
        float vreg[RIT][8], qv[RIT][8], kv[RIT][8], al[RIT][8], bet[RIT];
        float vmax = 0.f;
#pragma unroll
        for (int it = 0; it < RIT; ++it) {
            const int grp = wave + NW * it;
            if (grp >= RG) break;
            const int t = 4 * grp + lg;
            const bool rv = t < Lc;
            Vec8<Tin> rq, rk, rvv;
            Vec8<float> rg;
            float rb;
            if constexpr (PF) {
                rq.load((const Tin *)(sRaw + RL::Q) + t * kHeadDim + c8);
                rk.load((const Tin *)(sRaw + RL::K) + t * kHeadDim + c8);
                rvv.load((const Tin *)(sRaw + RL::V) + t * kHeadDim + c8);
                rg.load((const float *)(sRaw + RL::G) + t * kHeadDim + c8);
                rb = ((const float *)(sRaw + RL::B))[t];
            } else {
                const int tc = rv ? t : Lc - 1;
                const size_t row = (size_t)(t0c + tc) * H + h;
                const size_t rowk = (size_t)(t0c + tc) * p.Hk + h / (H / p.Hk);
                rq.load((const Tin *)p.q + rowk * kHeadDim + c8);
                rk.load((const Tin *)p.k + rowk * kHeadDim + c8);
                rvv.load((const Tin *)p.v + row * kHeadDim + c8);
                rg.load(p.g + row * kHeadDim + c8);
                rb = p.beta_raw[row];
            }
            // padding rows (t >= L, holding a copy of the last row) act as k = 0,
            // lambda = 0 and beta = 0: their rows of A, W and U_base are then zero
            // (T's row is beta_t e_t), so their q and v reach nothing that is
            // stored, and the chunk's total decay ignores them
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qv[it][e] = rq[e];
                kv[it][e] = rk[e];
                vreg[it][e] = rvv[e];
                sq += qv[it][e] * qv[it][e];
                sk += kv[it][e] * kv[it][e];
            }
            sq = row16_sum(sq);
            sk = row16_sum(sk);
            const float fq = rsqrtf(sq + kL2Eps) * p.scale, fk = rv ? rsqrtf(sk + kL2Eps) : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qv[it][e] *= fq;
                kv[it][e] *= fk;
                const float sg = fast_rcp(1.0f + fast_exp2(fmaf(rg[e], ga, gb[e])));
                al[it][e] = rv ? fast_exp2(lb2 * sg) : 1.f;
                vmax = fmaxf(vmax, fabsf(vreg[it][e]));
            }
            bet[it] = rv ? sigmoid_f(rb) : 0.f;
        }
        vmax = wave_max(vmax);
        if constexpr (PF) lds_barrier();       // all raw rows read before they are overwritten
#pragma unroll
        for (int it = 0; it < RIT; ++it) {
            const int grp = wave + NW * it;
            if (grp >= RG) break;
            const int t = 4 * grp + lg;
            *(f32x4 *)&sQ[t][c8] = f32x4{qv[it][0], qv[it][1], qv[it][2], qv[it][3]};
            *(f32x4 *)&sQ[t][c8 + 4] = f32x4{qv[it][4], qv[it][5], qv[it][6], qv[it][7]};
            *(f32x4 *)&sK[t][c8] = f32x4{kv[it][0], kv[it][1], kv[it][2], kv[it][3]};
            *(f32x4 *)&sK[t][c8 + 4] = f32x4{kv[it][4], kv[it][5], kv[it][6], kv[it][7]};
            *(f32x4 *)&sP[t][c8] = f32x4{al[it][0], al[it][1], al[it][2], al[it][3]};
            *(f32x4 *)&sP[t][c8 + 4] = f32x4{al[it][4], al[it][5], al[it][6], al[it][7]};
            if (lr == 0) sBeta[t] = bet[it];
        }
        if (lane == 0) sVmax[wave] = vmax;
        lds_barrier();

        // ---- phase 1b: block-local prefix products P_t = prod alpha_{16b+1 .. t};
        //      a thread per (16-row block, channel) also forms qh*P, kh*P and kh/P
        if (tid < NB * kHeadDim) {
            const int b = tid / kHeadDim, c = tid % kHeadDim;
            float a[16], kk[16], qq[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                a[i] = sP[16 * b + i][c];
                kk[i] = sK[16 * b + i][c];
                qq[i] = sQ[16 * b + i][c];
            }
            sA0[b][c] = a[0];
            float run = 1.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i > 0) run *= a[i];
                sQ[16 * b + i][c] = qq[i] * run;
                sK[16 * b + i][c] = kk[i] * run;
                sP[16 * b + i][c] = kk[i] * fast_rcp(run);
            }
            sPe[b][c] = run;
        }
        lds_barrier();

        // ---- phase 1c: per-channel block factors ---------------------------------
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
        if (tid == 0) sJob = 0;
        for (int idx = tid; idx < C * C; idx += NT) {   // zero the blocks of T above the diagonal
            const int i = idx / C, j = idx % C;
            if ((j >> 4) > (i >> 4)) sT[i][j] = 0.0f;
        }
        lds_barrier();

        // ---- phase 2: A and M blocks (MFMA); M, qg and kgT fragments -------------
        // Block (a, b), b <= a, of A = beta_i kh_i . kh_j e^{G_i - G_j} and of
        // M = qh_i . kh_j e^{G_i - G_j} is a K = 128 contraction of the rows of
        // qh*P / kh*P (block a) with kh/P (block b) scaled by the block factor EF
        // (a != b), computed transposed (M^T, A^T) so that the accumulator tile is
        // one half of M fragment (a, b / 2): block b fills positions 4 (b & 1) .. + 3
        // of each lane's 8 entries. Waves 0 .. NB-1 take the diagonal blocks (fp32
        // MFMA: right factors reach e^75) and invert I + A_aa; the other waves take
        // the off-diagonal blocks (fp16 MFMA: every factor is at most 1) and the qg
        // and kgT fragments.
        {
            auto block = [&](int a, int b) {
                const int il = 16 * a + lr, jr = 16 * b + lr;
                const float *ef = sEF[a > b ? a * (a - 1) / 2 + b : 0];
                f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aM = {0.f, 0.f, 0.f, 0.f};
                if (PRECISE || a == b) {
                    constexpr int KH = PRECISE ? 2 : 4;  // k-steps whose operands are loaded together
#pragma unroll
                    for (int k0 = 0; k0 < 4; k0 += KH) {
                        float bK[KH][8], bQ[KH][8], aR[KH][8];
#pragma unroll
                        for (int kq = 0; kq < KH; ++kq) {
                            const int c = 32 * (k0 + kq) + 8 * lg;
                            load8(&sK[il][c], bK[kq]);   // kh e^{G_i - G_16a}
                            load8(&sQ[il][c], bQ[kq]);   // qh e^{G_i - G_16a}
                            load8(&sP[jr][c], aR[kq]);   // kh / P_j
                            if (a != b) {                // e^{G_16a - G_j} = EF / P_j
                                float f[8];
                                load8(ef + c, f);
#pragma unroll
                                for (int e = 0; e < 8; ++e) aR[kq][e] *= f[e];
                            }
                        }
#pragma unroll
                        for (int kq = 0; kq < KH; ++kq) {
                            aA = mfma_f32x8(aR[kq], bK[kq], aA);
                            aM = mfma_f32x8(aR[kq], bQ[kq], aM);
                        }
                    }
                } else {
                    half8 hK[4], hQ[4], hR[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const int c = 32 * ks + 8 * lg;
                        float bK[8], bQ[8], aR[8], f[8];
                        load8(&sK[il][c], bK);
                        load8(&sQ[il][c], bQ);
                        load8(&sP[jr][c], aR);
                        load8(ef + c, f);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            hK[ks][e] = (_Float16)bK[e];
                            hQ[ks][e] = (_Float16)bQ[e];
                            hR[ks][e] = (_Float16)(aR[e] * f[e]);
                        }
                    }
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        aA = mfma_h(hR[ks], hK[ks], aA);
                        aM = mfma_h(hR[ks], hQ[ks], aM);
                    }
                }
                // lane holds A[i][j] / M[i][j] for i = 16a + lr, j = 16b + 4lg + ii
                float xm[8];
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int j = 16 * b + 4 * lg + ii;
                    sA[il][j] = (il > j) ? sBeta[il] * aA[ii] : 0.f;
                    xm[ii] = (j <= il) ? aM[ii] : 0.f;
                    xm[ii + 4] = 0.f;
                }
                unsigned char *mf = rec + R::M_OFF + ((size_t)(a * CS + (b >> 1)) * 64 + lane) * F::BYTES;
                if ((b & 1) == 0 && a == b) F::store(mf, xm);      // with the zero block b + 1
                else F::store_half(mf + (b & 1) * (F::BYTES / 2), xm);
            };

            if (wave < NB) {
                const int a = wave;
                block(a, a);
                // invert I + A_aa (strictly lower, written above by this wave; a
                // wave's LDS accesses complete in order, so the other lanes' entries
                // are visible to its later reads)
                const float *Ab = &sA[16 * a][16 * a];
                float *Xb = &sT[16 * a][16 * a];
                if constexpr (!PRECISE) {
                    // (I + A)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8) since A^16 = 0
                    float *Sx = &sX[a][0][0];
                    const f32x4 p1 = lds_right16(Ab, AP, lr, lg);
                    f32x4 z;
#pragma unroll
                    for (int i = 0; i < 4; ++i) z[i] = ((4 * lg + i == lr) ? 1.0f : 0.0f) - p1[i];
                    f32x4 pw = mm16(lds_left16(Ab, AP, lr, lg), p1, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int m = 0; m < 3; ++m) {
                        lds_store16(Sx, 20, pw, lr, lg);
                        const f32x4 lp = lds_left16(Sx, 20, lr, lg);
                        z = mm16(lp, z, z);                          // z += A^(2^(m+1)) z
                        if (m < 2) pw = mm16(lp, pw, f32x4{0.f, 0.f, 0.f, 0.f});
                    }
                    lds_store16(Xb, AP, z, lr, lg);
                } else if (lg == 0) {
                    // forward substitution, one column per lane (backward stable)
                    const int c = lr;
                    float x[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        float acc0 = (i == c) ? 1.0f : 0.0f, acc1 = 0.f;
#pragma unroll
                        for (int jj = 0; jj < i; jj += 2) {
                            acc0 -= Ab[i * AP + jj] * x[jj];
                            if (jj + 1 < i) acc1 -= Ab[i * AP + jj + 1] * x[jj + 1];
                        }
                        x[i] = (i < c) ? 0.0f : acc0 + acc1;
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) Xb[i * AP + c] = x[i];
                }
            }
            {
                // light jobs (off-diagonal blocks first, then the fragments), claimed
                // one at a time from a shared counter by whichever wave is free
                constexpr int NOFF = NB * (NB - 1) / 2;
                constexpr int NJ = NOFF + NB + 8;      // + qg row blocks + kg^T key blocks
                for (;;) {
                    int claim = 0;
                    if (lane == 0) claim = atomicAdd(&sJob, 1);
                    const int j = __builtin_amdgcn_readfirstlane(claim);
                    if (j >= NJ) break;
                    if (j < NOFF) {                      // off-diagonal block (a, b), a > b
                        const int a = j < 1 ? 1 : (j < 3 ? 2 : 3);
                        block(a, j - a * (a - 1) / 2);
                    } else if (j < NOFF + NB) {          // qg = qh e^{G_t} = (qh P_t) QF, rows of block tb
                        const int tb = j - NOFF;
                        const int t = 16 * tb + lr;
                        f32x4 q[8], f[8];
#pragma unroll
                        for (int h2 = 0; h2 < 8; ++h2) {     // channels 32 (h2/2) + 8 lg + 4 (h2%2) .. + 3
                            const int c = 32 * (h2 >> 1) + 8 * lg + 4 * (h2 & 1);
                            q[h2] = *(const f32x4 *)&sQ[t][c];
                            f[h2] = *(const f32x4 *)&sQF[tb][c];
                        }
#pragma unroll
                        for (int s = 0; s < 4; ++s) {        // fragment (tb, s): channels 32 s + 8 lg + e
                            float x[8];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                x[e] = q[2 * s][e] * f[2 * s][e];
                                x[e + 4] = q[2 * s + 1][e] * f[2 * s + 1][e];
                            }
                            F::store(rec + R::QG_OFF + ((size_t)(tb * 4 + s) * 64 + lane) * F::BYTES, x);
                        }
                    } else {                             // kg = kh e^{G_C - G_t} = (kh / P_t) KF
                        const int kb = j - NOFF - NB;
                        const int c = tile_chan(kb, lr);
                        float x[CS][8];
#pragma unroll
                        for (int s = 0; s < CS; ++s)
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const int t = 32 * s + kperm(lg, e);
                                x[s][e] = (t < C) ? sP[t][c] * sKF[t >> 4][c] : 0.f;
                            }
#pragma unroll
                        for (int s = 0; s < CS; ++s)
                            F::store(rec + R::KG_OFF + ((size_t)(kb * CS + s) * 64 + lane) * F::BYTES, x[s]);
                    }
                }
            }
        }
        // power-of-two scale of v for the fp16 product T v (exact)
        float vscale = 1.0f;
        bool vinv_zero = false;                   // all v of the chunk are zero: Ub = 0
        if constexpr (!PRECISE) {
            float m = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) m = fmaxf(m, sVmax[w]);
            vscale = pow2_scale_for(m, 9);          // |T v / vscale| <= 64 * 2^9 = 2^15
            vinv_zero = !(m > 0.f);
        }
        const float vinv = inv_pow2(vscale);
        lds_barrier();
        // the qh*P tile is free from here on: the next tile's q and k go there
        if constexpr (PF) {
            static_assert(RawLayout<C, Tin>::V <= sizeof(float) * C * KP, "q, k fit the qh*P tile");
            if (valid_nx) stage_raw<C, Tin, 0>(p, (int)(next % H), t0_nx, L_nx, tid, sRaw);
        }

        // ---- phase 3: v (scaled) into sP ----------------------------------------
#pragma unroll
        for (int it = 0; it < RIT; ++it) {
            const int grp = wave + NW * it;
            if (grp >= RG) break;
            const int t = 4 * grp + lg;
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = vreg[it][e] * vinv;
            *(f32x4 *)&sP[t][c8] = f32x4{x[0], x[1], x[2], x[3]};
            *(f32x4 *)&sP[t][c8 + 4] = f32x4{x[4], x[5], x[6], x[7]};
        }
        if (tid == 0) *(float *)(rec + R::UBS_OFF) = (vinv_zero ? 0.0f : vscale);
        lds_barrier();

        // phase-5 operands that do not depend on T, built before the inverse ends:
        // W^T A operand (kh e^{G_j} = (kh P_j) QF, channel tiles 2s', 2s'+1 with
        // s' = wave % 4) and the Ub B operand (v columns of block vb = wave).
        const int sw = wave & 3;
        const int ca = tile_chan(2 * sw, lr), cb = tile_chan(2 * sw + 1, lr);
        const int col = 16 * wave + lr;
        float a0[CS][8], a1[CS][8], bV[CS][8];
#pragma unroll
        for (int sp = 0; sp < CS; ++sp)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int jx = 32 * sp + 8 * lg + e;
                const bool in = jx < C;
                const int bj = in ? (jx >> 4) : 0;
                a0[sp][e] = in ? sK[jx][ca] * sQF[bj][ca] : 0.f;
                a1[sp][e] = in ? sK[jx][cb] * sQF[bj][cb] : 0.f;
                bV[sp][e] = in ? sP[jx][col] : 0.f;
            }

        // next tile: its raw inputs load during the inverse and the W / Ub products
        ti = next;
        valid = valid_nx;
        n = n_nx;
        t0 = t0_nx;
        L = L_nx;
        if constexpr (PF) {
            lds_barrier();                      // the three tiles are free from here on
            if (valid) stage_raw<C, Tin, 1>(p, (int)(ti % H), t0, L, tid, sRaw);
        }

        // ---- phase 4: off-diagonal blocks X_ab = -X_aa sum_{c=b}^{a-1} A_ac X_cb ----
        // in two levels of independent 16x16 fp32 MFMA chains (products feed the
        // next one from registers): first X_10 and X_32, then, with
        // Y_rc = A_r0 X_0c + A_r1 X_1c (X_01 = 0), X_2c = -X_22 Y_2c and
        // X_3c = -(X_32 Y_2c + X_33 Y_3c), which is the substitution above with
        // X_32 = -X_33 A_32 X_22 folded in.
        if constexpr (NB >= 2) {
            if (wave < NB / 2) {
                const int a = 2 * wave + 1, b = 2 * wave;
                const f32x4 y = mm16(lds_left16(&sA[16 * a][16 * b], AP, lr, lg),
                                     lds_right16(&sT[16 * b][16 * b], AP, lr, lg), f32x4{0.f, 0.f, 0.f, 0.f});
                const f32x4 x = mm16(lds_left16(&sT[16 * a][16 * a], AP, lr, lg), y, f32x4{0.f, 0.f, 0.f, 0.f});
                lds_store16(&sT[16 * a][16 * b], AP, -x, lr, lg);
            }
            lds_barrier();
        }
        if constexpr (NB == 4) {
            if (wave < 4) {
                const int r = 2 + (wave >> 1), c = wave & 1;
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const f32x4 x1c = lds_right16(&sT[16][16 * c], AP, lr, lg);    // X_1c
                f32x4 x00 = zero;
                if (c == 0) x00 = lds_right16(&sT[0][0], AP, lr, lg);
                f32x4 y2 = mm16(lds_left16(&sA[32][16], AP, lr, lg), x1c, zero);            // A_21 X_1c
                if (c == 0) y2 = mm16(lds_left16(&sA[32][0], AP, lr, lg), x00, y2);         // + A_20 X_00
                f32x4 x;
                if (r == 2) {
                    x = mm16(lds_left16(&sT[32][32], AP, lr, lg), y2, zero);                // X_22 Y_2c
                } else {
                    f32x4 y3 = mm16(lds_left16(&sA[48][16], AP, lr, lg), x1c, zero);        // A_31 X_1c
                    if (c == 0) y3 = mm16(lds_left16(&sA[48][0], AP, lr, lg), x00, y3);     // + A_30 X_00
                    x = mm16(lds_left16(&sT[48][32], AP, lr, lg), y2, zero);                // X_32 Y_2c
                    x = mm16(lds_left16(&sT[48][48], AP, lr, lg), y3, x);                   // + X_33 Y_3c
                }
                lds_store16(&sT[16 * r][16 * c], AP, -x, lr, lg);
            }
            lds_barrier();
        }

        // ---- phase 5: W^T = (kh e^G)^T T^T and Ub = T v (MFMA) --------------------
        // Results stay in registers until the next tile's copies have landed, so
        // that the wait below does not also wait for these stores.
        float wres[2][8];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
            const int tb = 2 * (wave >> 2) + q2;
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            if (tb < NB) {
                const int i = 16 * tb + lr;
#pragma unroll
                for (int sp = 0; sp < CS; ++sp) {
                    if (32 * sp > 16 * tb + 15) continue;      // T is lower triangular
                    float bT[8];
                    const int j0 = 32 * sp + 8 * lg;
                    if (j0 < C) load_T_row(&sT[i][j0], &sBeta[j0], bT);     // T = X diag(beta)
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
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) { wres[q2][e] = acc0[e]; wres[q2][e + 4] = acc1[e]; }
        }
        f32x4 ures[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            const int i = 16 * tb + lr;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sp = 0; sp < CS; ++sp) {
                if (32 * sp > 16 * tb + 15) continue;
                float aT[8];
                const int j0 = 32 * sp + 8 * lg;
                if (j0 < C) load_T_row(&sT[i][j0], &sBeta[j0], aT);
                else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) aT[e] = 0.f;
                }
                if constexpr (PRECISE) acc = mfma_f32x8(aT, bV[sp], acc);
                else acc = mfma_f16(aT, bV[sp], acc);
            }
            ures[tb] = acc;
        }
        if constexpr (PF) wait_vmem();        // the next tile's inputs have landed
        lds_barrier();                      // LDS is reused by the next tile
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {        // W stored negated: U = Ub + (-W) S^T
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = -wres[q2][e];
            pend_w[q2] = F::make(x, 1.0f);
        }
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            if constexpr (PRECISE) pend_u[tb] = ures[tb];
            else pend_u[tb] = half4_t{(_Float16)ures[tb][0], (_Float16)ures[tb][1],
                                      (_Float16)ures[tb][2], (_Float16)ures[tb][3]};
        }
        pend_rec = rec;
    }
    flush();
}

// =============================================================================
// Inter-chunk kernel: two workgroups (4 waves each) per (sequence, head), one
// per 64-row half of the state; each wave owns 16 state rows, held in
// registers as S^T accumulator tiles. The per-chunk operands are copied
// global -> LDS by the DMA path (no register staging), one chunk ahead into a
// second buffer when two fit.
// =============================================================================
template <int C, bool PRECISE, int D = 128>
struct InterCfg {
    using R = Record<C, PRECISE, D>;
    static constexpr int SH_BLOCKS = (int)((R::SHARED_BYTES + 1023) / 1024);   // 1 KiB copies
    static constexpr size_t UB_LDS = (size_t)SH_BLOCKS * 1024;   // this half's Ub in LDS
    static constexpr int UB_BLOCKS = (int)(4 * R::UB_VB_BYTES / 1024);
    static constexpr int BLOCKS = SH_BLOCKS + UB_BLOCKS;
    static constexpr size_t BUF = (size_t)BLOCKS * 1024;
    static constexpr int NBUF = (2 * BUF <= 160 * 1024) ? 2 : 1;
    static_assert(4 * R::UB_VB_BYTES % 1024 == 0, "the Ub half is whole 1 KiB blocks");
    // The last shared block reads past SHARED_BYTES into the record's own Ub area.
    static_assert(UB_LDS <= R::BYTES, "shared-block over-read stays inside the record");
};

template <typename T> __device__ __forceinline__ void store4(T *p, const f32x4 &x);
template <> __device__ __forceinline__ void store4<float>(float *p, const f32x4 &x) {
    *(f32x4 *)p = x;
}
template <> __device__ __forceinline__ void store4<__bf16>(__bf16 *p, const f32x4 &x) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    *(bf16x4 *)p = bf16x4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
}

// Polls of the other half's row sums before a fused epilogue gives up (about a
// second): the workgroup's outputs are then NaN rather than a hang.
constexpr int kXchgSpin = 1 << 20;

// GATE (64-row chunks of bf16 inputs, D = 128): the output epilogue fused in
// (kimi_k3 FusedKDAChunkwise page, "Output handling": per-row RMS norm over the
// 128 features, channel weight, sigmoid output gate). A row's features come
// from the two workgroups of its chain, 64 each, so its sum of squares is
// completed across them. A fifth wave per workgroup does that, one chunk step
// behind the four state waves each time:
//   step j     the state waves leave chunk j's partial sums of squares in LDS
//              and keep its outputs x = O sigma in registers;
//   step j + 1 the fifth wave adds up this half's sums and posts them for the
//              other workgroup (a (sum, tag) word per row in the workspace,
//              zeroed before the launch);
//   step j + 2 it asks for the other half's sums (posted a step earlier) and
//              loads the chunk's gate logits;
//   step j + 3 it forms r = 1 / sqrt(mean(o^2) + eps) per row and leaves r and
//              the logits in LDS;
//   step j + 4 the state waves store y = x r w sigmoid(z).
// Every load has a whole step to arrive: the exchange goes through the
// device-coherent level of the memory hierarchy (the two workgroups need not
// share an L2). The two workgroups of a chain must be resident at the same
// time: the launch keeps the whole grid within one round of workgroups.
template <int C, typename Tout, bool PRECISE, int D = 128, bool GATE = false>
__global__ __launch_bounds__(GATE ? 320 : 256) void inter_kernel(PrefillArgs p, int nchains)
{
    using G = ChunkGeom<C>;
    using R = Record<C, PRECISE, D>;
    using F = Frag<PRECISE>;
    using FT = typename F::T;
    using CFG = InterCfg<C, PRECISE, D>;
    constexpr int NB = G::NB, CS = G::CS;
    constexpr int KS = R::KS, KT = R::KT;
    constexpr int HALVES = D / 64;                  // workgroups (64 state rows each) per chain
    extern __shared__ __align__(16) unsigned char smem[];

    // workgroup -> (chain, half); both halves of a chain land on the same XCD
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    int chain = (local / HALVES) * 8 + xcd;
    const int vg = local % HALVES;
    if (chain >= nchains) return;
    const int H = p.H;
    int n = chain / H;
    const int h = chain % H;
    // Packed batches of up to 64 sequences take them longest first: the chains
    // of rank r go to the r-th row of workgroups, so the longest chains start
    // in the first round of workgroups (one per CU) and shorter ones fill in
    // behind them instead of trailing at the end. Lane m ranks sequence m by
    // length (ties by index); the lane holding rank n names the sequence.
    if (p.N > 1 && p.N <= 64) {
        const int lane = threadIdx.x & 63;
        int rank = -1;
        if (lane < p.N) {
            const int64_t len_l = p.cu_seqlens[lane + 1] - p.cu_seqlens[lane];
            rank = 0;
            for (int m = 0; m < p.N; ++m) {
                const int64_t len_m = p.cu_seqlens[m + 1] - p.cu_seqlens[m];
                rank += (len_m > len_l || (len_m == len_l && m < lane)) ? 1 : 0;
            }
        }
        const uint64_t hit = __builtin_amdgcn_ballot_w64(rank == n);
        n = hit ? (int)__builtin_ctzll(hit) : n;       // ranks are a permutation: one lane
        chain = n * H + h;
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lr = lane & 15, lg = lane >> 4;
    const int vb = 4 * vg + wave;
    const int vrow = 16 * vb + lr;               // this lane's state row

    const int64_t s0 = p.cu_seqlens[n];
    const int64_t len = p.cu_seqlens[n + 1] - s0;
    const int nch = (int)((len + C - 1) / C);
    const int64_t slot0 = s0 / C + n;

    // fused epilogue, after the record buffers: the state waves' partial row
    // sums [2][64 rows][4 waves][4 column groups], the rows' inverse rms
    // [2][64] and a chunk's gate logits for this half [2][64 rows][64] (bf16)
    float *const ssw = (float *)(smem + CFG::NBUF * CFG::BUF);
    float *const rinv = ssw + 2 * 64 * 16;
    unsigned char *const szb = (unsigned char *)(rinv + 2 * 64);
    if constexpr (GATE) {
        static_assert(D == 128 && HALVES == 2 && CFG::NBUF == 2, "fused epilogue: two halves, two buffers");
        if (wave == 4) {
            // The fifth wave: one barrier per state-wave step 0 .. nch + 2 (the
            // state waves' last step, nch + 3, has none). In step jc it posts this
            // half's row sums of chunk jc - 1 and asks for the other half's of
            // chunk jc - 2 (posted a step earlier); in step jc + 1 it forms their
            // r from the answer and leaves chunk jc - 2's gate logits in LDS.
            // (Forming sigmoid(z) here measured slower: this wave shares a SIMD
            // with a state wave, whose arithmetic it then delays.) Every step issues the
            // same loads and stores (steps without a chunk use chunk 0 and a
            // spare word), so that the waits the compiler places for them count
            // right and leave them in flight across the step.
            if (nch <= 0) return;
            lds_barrier();
            uint64_t *const xc = p.xchg + ((size_t)slot0 * H + h) * 128 + lane;
            const size_t xstep = (size_t)H * 128;
            uint64_t *const spare = (uint64_t *)(p.ws + (size_t)num_slots(p.T, p.N, C) * H * R::BYTES + 128);
            bool gave_up = false;       // after one wait ran out, no more waiting
            // gate rows of a chunk, eight per load: lane holds row 8 c + lane / 8,
            // columns 8 (lane % 8) .. + 7 of this half
            i32x4 zv[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) zv[c] = i32x4{0, 0, 0, 0};
            uint64_t other = 0;
            float own_a = 0.f, own_b = 0.f;     // this half's sums of chunks jc - 3, jc - 2
            for (int jc = 0; jc <= nch + 2; ++jc) {
                // chunk jc - 3's gate, loaded in the last step, into LDS buffer (jc - 3) & 1
                unsigned char *const dst = szb + ((jc + 1) & 1) * 8192 + 16 * lane;
#pragma unroll
                for (int c = 0; c < 8; ++c) *(i32x4 *)(dst + 1024 * c) = zv[c];
                // r of chunk jc - 3 from the other half's answer
                if (jc >= 3) {
                    const int j = jc - 3;
                    const uint32_t tag = (uint32_t)j + 1u;
                    if (__builtin_amdgcn_ballot_w64((uint32_t)(other >> 32) != tag) != 0) {
                        const uint64_t *const eo = xc + (size_t)j * xstep + 64 * (vg ^ 1);
                        for (int it = 0;; ++it) {
                            if (gave_up || it >= kXchgSpin) { other = 0x7fc00000u; gave_up = true; break; }
                            __builtin_amdgcn_s_sleep(1);
                            other = __hip_atomic_load(eo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            if (__builtin_amdgcn_ballot_w64((uint32_t)(other >> 32) != tag) == 0) break;
                        }
                    }
                    const float ot = __uint_as_float((uint32_t)other);
                    const float tot = vg == 0 ? own_a + ot : ot + own_a;   // the same order in both
                    rinv[(j & 1) * 64 + lane] = rsqrtf(tot * (1.0f / D) + p.norm_eps);
                }
                // the other half's sums of chunk jc - 2, asked for
                const int jo = jc >= 2 ? jc - 2 : 0;
                other = __hip_atomic_load(xc + (size_t)jo * xstep + 64 * (vg ^ 1), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                // chunk jc - 2's gate logits (rows past the sequence end repeat its last row)
                const int64_t t0 = (int64_t)(jc < 2 ? 0 : (jc - 2 < nch ? jc - 2 : nch - 1)) * C;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int64_t t = t0 + 8 * c + (lane >> 3);
                    zv[c] = *(const i32x4 *)((const __bf16 *)p.z + ((size_t)(s0 + (t < len ? t : len - 1)) * H + h) * D +
                                             64 * vg + 8 * (lane & 7));
                }
                // this half's sums of chunk jc - 1, posted
                const int jp = jc - 1;
                const f32x4 *const pw = (const f32x4 *)(ssw + ((jp & 1) * 64 + lane) * 16);
                f32x4 ps[4];
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) ps[w4] = pw[w4];     // state wave w4's four column groups
                float own = 0.f;
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) own += (ps[w4][0] + ps[w4][1]) + (ps[w4][2] + ps[w4][3]);
                __hip_atomic_store(jc >= 1 && jc <= nch ? xc + (size_t)jp * xstep + 64 * vg : spare,
                                   ((uint64_t)(jp + 1) << 32) | __float_as_uint(own),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                own_a = own_b;
                own_b = own;
                lds_barrier();
            }
            return;
        }
    }

    // State S^T tiles: lane holds S[vrow][tile_chan(kb, 4 lg + i)] (the row order
    // of the kg^T tiles it accumulates from). On the fp16 path the
    // registers hold S / sigma for a wave-uniform power of two sigma, chosen so
    // that S / sigma converts to fp16 without overflow and U / sigma too.
    f32x4 S[KT];
    float sigma = 1.0f;
    const size_t sbase = ((size_t)chain * D + vrow) * D;
#pragma unroll
    for (int kb = 0; kb < KT; ++kb) S[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.h0) {
#pragma unroll
        for (int kb = 0; kb < KT; ++kb) S[kb] = *(const f32x4 *)(p.h0 + sbase + tile_chan(kb, 4 * lg));
    }

    // DMA copy of chunk jc's record into LDS buffer buf, in parts spread over
    // the chunk: the shared operands, then this half's Ub blocks; wave w copies
    // the 1 KiB blocks w, w + 4, ... through a buffer resource covering exactly
    // the record, with the wave-uniform part of each offset in soffset.
    constexpr int SHI = (CFG::SH_BLOCKS + 3) / 4, UBI = (CFG::UB_BLOCKS + 3) / 4;
    constexpr int NCP = SHI + UBI;
    const unsigned char *rec0 = p.ws + ((size_t)slot0 * H + h) * R::BYTES;
    const size_t rec_step = (size_t)H * R::BYTES;
    const uint32_t lane16 = 16u * (uint32_t)lane;
    const uint32_t ub_off = (uint32_t)(R::UB_OFF + (size_t)4 * vg * R::UB_VB_BYTES);
    auto fetch = [&](int jc, int buf, int k0, int k1) {
        const i32x4 r = make_rsrc(rec0 + (size_t)jc * rec_step, (uint32_t)R::BYTES);
        unsigned char *dst = smem + (size_t)buf * CFG::BUF + 1024 * wave;
#pragma unroll
        for (int k = 0; k < NCP; ++k) {
            if (k < k0 || k >= k1) continue;
            if (k < SHI) {
                if (4 * k + 3 < CFG::SH_BLOCKS || 4 * k + wave < CFG::SH_BLOCKS)
                    copy16_to_lds(r, lane16, 1024u * wave + 4096u * k, dst + 4096 * k);
            } else {
                const int i = k - SHI;
                if (4 * i + 3 < CFG::UB_BLOCKS || 4 * i + wave < CFG::UB_BLOCKS)
                    copy16_to_lds(r, lane16, ub_off + 1024u * wave + 4096u * i,
                                  dst + CFG::UB_LDS + 4096 * i);
            }
        }
    };

    // L2 prefetch two chunks ahead: one 4-byte load per 128-byte line of this
    // workgroup's share of a record (the two halves of a chain split the shared
    // operands). The values are never used; they stay in registers until the
    // end-of-chunk wait so that no earlier wait is placed on them. Every lane
    // issues every load (lanes past the share re-touch line 0), so that each
    // wave issues the same known number of memory instructions per chunk.
    constexpr int SHL = (int)((R::SHARED_BYTES + 127) / 128), SHL2 = (SHL + HALVES - 1) / HALVES;
    constexpr int UBL = (int)(4 * R::UB_VB_BYTES / 128);
    constexpr int NTOUCH = (SHL2 + UBL + 255) / 256;
    uint32_t touch_off[NTOUCH];
#pragma unroll
    for (int i = 0; i < NTOUCH; ++i) {
        const int li = tid + 256 * i;
        const int sh = vg * SHL2 + li;
        touch_off[i] = (li < SHL2) ? ((sh < SHL) ? 128u * sh : 0u)
                     : (li < SHL2 + UBL ? ub_off + 128u * (li - SHL2) : 0u);
    }
    uint32_t touched[NTOUCH];
#pragma unroll
    for (int i = 0; i < NTOUCH; ++i) touched[i] = 0;
    auto touch = [&](int jc) {
        const unsigned char *r = rec0 + (size_t)jc * rec_step;
#pragma unroll
        for (int i = 0; i < NTOUCH; ++i) touched[i] = *(const uint32_t *)(r + touch_off[i]);
    };

    // this lane writes o[t][h][16 vb + 4 lg .. + 3] for t = chunk start + 16 tb + lr,
    // at the end of the chunk; lanes whose row lies past the sequence end write
    // the same 16 bytes of the workspace's spare tail instead, so that every
    // lane issues every store (the end-of-chunk wait counts them)
    Tout *__restrict__ o = (Tout *)p.o + ((size_t)(s0 + lr) * H + h) * D + 16 * vb + 4 * lg;
    Tout *const o_spare = (Tout *)(p.ws + (size_t)num_slots(p.T, p.N, C) * H * R::BYTES);
    const size_t o_tb = (size_t)16 * H * D, o_chunk = (size_t)C * H * D;
    // fp16 outputs (staged for the output epilogue): each row's 16-value block
    // vb is stored divided by a power-of-two scale (its largest magnitude below
    // 2^15, so no overflow and half an fp16 ulp of the block's largest value),
    // the scale in o_scale[row][vb]; the spare tail takes the scales of rows
    // past the sequence end too
    constexpr bool SCALED = std::is_same<Tout, _Float16>::value;
    static_assert(!(SCALED && GATE), "the fused epilogue stores bf16 or fp32");
    // fused epilogue: chunk j's outputs x (O sigma) wait four steps in xa .. xd
    // (xn: the step's new chunk; a loop unrolled four times, which would keep
    // them in place, needs more than the 256 registers); the lane's four
    // columns 16 vb + 4 lg + i of the norm weight
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    [[maybe_unused]] f32x4 xa[NB], xb[NB], xc[NB], xd[NB], xn[NB], wv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) xa[tb] = xb[tb] = xc[tb] = xd[tb] = xn[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (GATE) wv = *(const f32x4 *)(p.norm_w + 16 * vb + 4 * lg);
    float *__restrict__ osc = SCALED ? p.o_scale + ((size_t)(s0 + lr) * H + h) * (D / 16) + vb : nullptr;
    float *const osc_spare = (float *)o_spare + 16;
    const size_t osc_tb = (size_t)16 * H * (D / 16), osc_chunk = (size_t)C * H * (D / 16);

    if (nch > 0) {
        fetch(0, 0, 0, NCP);
        if (nch > 1) touch(1);
        wait_vmem();
        lds_barrier();
    }
    // with the fused epilogue four more steps store the last four chunks' rows
    const int nsteps = GATE ? (nch > 0 ? nch + 4 : 0) : nch;
    for (int jc = 0; jc < nsteps; ++jc) {
        const int buf = (CFG::NBUF == 2) ? (jc & 1) : 0;
        const bool ahead = CFG::NBUF == 2 && jc + 1 < nch;
        const unsigned char *B = smem + (size_t)buf * CFG::BUF;
        const int L = (len - (int64_t)jc * C) < C ? (int)(len - (int64_t)jc * C) : C;
        if (ahead) fetch(jc + 1, buf ^ 1, 0, NCP);
        [[maybe_unused]] float ry[NB];
        [[maybe_unused]] bf16x4_t zy[NB];
        if constexpr (GATE) {
            touch(jc + 2 < nch ? jc + 2 : nch - 1);   // every step issues the same loads
            // r and z of the rows of chunk jc - 4, for the step's end
            const int jy = jc - 4;
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                ry[tb] = rinv[(jy & 1) * 64 + 16 * tb + lr];
                zy[tb] = *(const bf16x4_t *)(szb + (jy & 1) * 8192 + (16 * tb + lr) * 128 + 32 * wave + 8 * lg);
            }
        } else {
            touch(jc + 2 < nch ? jc + 2 : jc);
        }
        if (!GATE || jc < nch) {

        // operands are requested one 16-row tile ahead of the products using them
        auto frag = [&](size_t off, int idx) { return F::load(B + off + ((size_t)idx * 64 + lane) * F::BYTES); };
        FT fw[2][KS], fq[2][KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) { fw[0][s] = frag(R::W_OFF, s); fq[0][s] = frag(R::QG_OFF, s); }
        f32x4 ub[NB];
        float us = 1.0f;
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            const unsigned char *ubp = B + CFG::UB_LDS +
                                       ((size_t)(wave * NB + tb) * 64 + lane) * 4 * R::UB_ELT;
            if constexpr (PRECISE) {
                ub[tb] = *(const f32x4 *)ubp;
            } else {
                typedef _Float16 half4 __attribute__((ext_vector_type(4)));
                const half4 hv = *(const half4 *)ubp;
#pragma unroll
                for (int i = 0; i < 4; ++i) ub[tb][i] = (float)hv[i];
            }
        }
        if constexpr (!PRECISE) us = *(const float *)(B + R::UBS_OFF);


        // rescale the state when S / sigma leaves [2^4, 2^14] or sigma < us
        // (|Ub| / sigma <= 2^15 needs sigma >= us); both are powers of two
        // (the wave maximum is formed only when a lane's own maximum says that
        // a rescale may be due: two ballots instead of a reduction per chunk)
        if constexpr (!PRECISE) {
            float m = 0.f;
#pragma unroll
            for (int kb = 0; kb < KT; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[kb][i]));
            const bool any_big = __builtin_amdgcn_ballot_w64(m > 16384.f) != 0;
            const bool all_small = __builtin_amdgcn_ballot_w64(!(m < 16.f)) == 0;
            if (any_big || all_small || sigma < us) {
                m = wave_max_nonneg(m);
                float tgt = (m > 0.f) ? sigma * pow2_scale_for(m, 14) : (us > 0.f ? us : sigma);
                if (tgt < us) tgt = us;
                if (m > 16384.f || sigma < us || (m < 16.f && tgt < sigma)) {
                    const float r = sigma / tgt;
#pragma unroll
                    for (int kb = 0; kb < KT; ++kb) S[kb] *= r;
                    sigma = tgt;
                }
            }
        }
        // state operand: k-step s covers channels 32 s + 8 lg + e (tiles 2s, 2s+1); it is the
        // B operand of W S^T (columns v) and the A operand of S qg^T (rows v)
        FT bS[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            float x[8] = {S[2 * s][0], S[2 * s][1], S[2 * s][2], S[2 * s][3],
                          S[2 * s + 1][0], S[2 * s + 1][1], S[2 * s + 1][2], S[2 * s + 1][3]};
            bS[s] = F::make(x, 1.0f);
        }

        // U / sigma = Ub / sigma + (-W) S^T / sigma  (tile [t][v]: t = 16 tb + 4 lg + i, v = vrow)
        // O / sigma = S qg^T / sigma                 (tile [v][t]: v = 16 vb + 4 lg + i, t = 16 tb + lr)
        const float ubf = us / sigma;
        f32x4 U[NB], O[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            if (tb + 1 < NB) {
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    fw[(tb + 1) & 1][s] = frag(R::W_OFF, (tb + 1) * KS + s);
                    fq[(tb + 1) & 1][s] = frag(R::QG_OFF, (tb + 1) * KS + s);
                }
            }
            f32x4 aw = ub[tb] * ubf, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                aw = F::mma(fw[tb & 1][s], bS[s], aw);
                aq = F::mma(bS[s], fq[tb & 1][s], aq);
            }
            U[tb] = aw;
            O[tb] = aq;
        }

        // operands of the second products: M, then kg^T two key blocks ahead
        FT fm[NB][CS], fk[3][CS];
        f32x4 gv[KT];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
#pragma unroll
            for (int s = 0; s < CS; ++s)
                if (32 * s <= 16 * tb + 15)                // M is lower triangular
                    fm[tb][s] = frag(R::M_OFF, tb * CS + s);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s = 0; s < CS; ++s) fk[kb][s] = frag(R::KG_OFF, kb * CS + s);
#pragma unroll
        for (int kb = 0; kb < KT; ++kb) gv[kb] = *(const f32x4 *)(B + R::GC_OFF + 4 * tile_chan(kb, 4 * lg));

        // U / sigma must fit fp16: otherwise raise sigma (rare)
        if constexpr (!PRECISE) {
            float m = 0.f;
#pragma unroll
            for (int tb = 0; tb < NB; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(U[tb][i]));
            if (__builtin_amdgcn_ballot_w64(m > 32768.f) != 0) {
                m = wave_max_nonneg(m);
                const float f = pow2_scale_for(m, 14), r = inv_pow2(f);
#pragma unroll
                for (int tb = 0; tb < NB; ++tb) { U[tb] *= r; O[tb] *= r; }
#pragma unroll
                for (int kb = 0; kb < KT; ++kb) S[kb] *= r;
                sigma *= f;
            }
        }
        // U operand: k-step s over t covers rows 32 s + kperm(lg, e); it is the
        // B operand of kg^T U (columns v) and the A operand of U^T M^T (rows v)
        FT bU[CS];
#pragma unroll
        for (int s = 0; s < CS; ++s) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = (2 * s < NB) ? U[2 * s][e] : 0.f;
                x[e + 4] = (2 * s + 1 < NB) ? U[2 * s + 1][e] : 0.f;
            }
            bU[s] = F::make(x, 1.0f);
        }

        // O^T += U^T M^T
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
#pragma unroll
            for (int s = 0; s < CS; ++s)
                if (32 * s <= 16 * tb + 15) O[tb] = F::mma(bU[s], fm[tb][s], O[tb]);

        // S^T <- diag(GamC) S^T + kg^T U
#pragma unroll
        for (int kb = 0; kb < KT; ++kb) {
            if (kb + 2 < KT) {
#pragma unroll
                for (int s = 0; s < CS; ++s) fk[(kb + 2) % 3][s] = frag(R::KG_OFF, (kb + 2) * CS + s);
            }
            f32x4 acc = S[kb] * gv[kb];
#pragma unroll
            for (int s = 0; s < CS; ++s) acc = F::mma(fk[kb % 3][s], bU[s], acc);
            S[kb] = acc;
        }

        if constexpr (GATE) {
            // keep x, leave its rows' 16-column sums of squares for the fifth wave
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                const f32x4 x = O[tb] * sigma;
                xn[tb] = x;
                ssw[((jc & 1) * 64 + 16 * tb + lr) * 16 + 4 * wave + lg] =
                    (x[0] * x[0] + x[1] * x[1]) + (x[2] * x[2] + x[3] * x[3]);
            }
        } else if constexpr (SCALED) {
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                const f32x4 x = O[tb] * sigma;
                // largest magnitude of the row's block: the lane's four values, then
                // the four lanes lr + 16 lg holding the block's other values
                float m = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
                const auto a32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
                m = fmaxf(__uint_as_float(a32[0]), __uint_as_float(a32[1]));
                const auto a16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
                m = fmaxf(__uint_as_float(a16[0]), __uint_as_float(a16[1]));
                const float sc = pow2_scale_for(m, 15), inv = inv_pow2(sc);
                const bool in = 16 * tb + lr < L;
                *(half4_t *)(in ? o + tb * o_tb : o_spare) =
                    half4_t{(_Float16)(x[0] * inv), (_Float16)(x[1] * inv), (_Float16)(x[2] * inv), (_Float16)(x[3] * inv)};
                *(in ? osc + tb * osc_tb : osc_spare) = sc;   // the four lanes of a block store the same value
            }
            osc += osc_chunk;
        } else {
#pragma unroll
            for (int tb = 0; tb < NB; ++tb)
                store4<Tout>(16 * tb + lr < L ? o + tb * o_tb : o_spare, O[tb] * sigma);
        }
        if constexpr (!GATE) o += o_chunk;
        }   // the chunk's products
        if constexpr (GATE) {
            // rows of chunk jc - 4: y = x r w sigmoid(z), r and z (read at the
            // step start) left by the fifth wave
            const int jy = jc - 4;
            const int Ly = jy < 0 ? 0 : ((len - (int64_t)jy * C) < C ? (int)(len - (int64_t)jy * C) : C);
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                f32x4 y;
#pragma unroll
                for (int i = 0; i < 4; ++i)     // sigmoid as 1 / (1 + 2^(-z log2 e)): 0 and 1 at the ends
                    y[i] = xa[tb][i] * ry[tb] * wv[i] * fast_rcp(1.0f + fast_exp2(-kLog2e * (float)zy[tb][i]));
                store4<Tout>(16 * tb + lr < Ly ? o + (size_t)jy * o_chunk + tb * o_tb : o_spare, y);
            }
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) { xa[tb] = xb[tb]; xb[tb] = xc[tb]; xc[tb] = xd[tb]; xd[tb] = xn[tb]; }
            // the copies issued at the step start have landed; the NB output
            // stores issued after them may still be in flight
            if (jc + 1 < nch) wait_vmem_except<NB>();
            if (jc <= nch + 2) lds_barrier();
        } else if (jc + 1 < nch) {
            if (CFG::NBUF == 1) {
                lds_barrier();            // everyone is done with the single buffer
                fetch(jc + 1, 0, 0, NCP);
                wait_vmem();
            } else {
                // the copies and touches issued at the chunk start have landed; the
                // output stores issued since (the newest) may still be in flight
                wait_vmem_except<(SCALED ? 2 : 1) * NB>();
            }
            lds_barrier();                // ... and everyone else's
        }
#pragma unroll
        for (int i = 0; i < NTOUCH; ++i) asm volatile("" ::"v"(touched[i]));
    }

    if (p.ht) {
#pragma unroll
        for (int kb = 0; kb < KT; ++kb)
            *(f32x4 *)(p.ht + sbase + tile_chan(kb, 4 * lg)) = S[kb] * sigma;
    }
}

// =============================================================================
// Intra-chunk kernel for 64-row chunks with bf16 inputs (fp16 records): four
// waves per workgroup, wave b holding rows 16b .. 16b+15 of the tile in
// registers in the MFMA operand layout -- lane (lr, lg) holds row lr at the key
// channels 32 s + 8 lg + e, s = 0..3, e = 0..7 (16 contiguous bytes of a bf16
// row per k-step, one load each) -- so that the norms, gates
// and decay factors are computed where the products consume them. About 74 KiB
// of LDS, so two workgroups share a CU and one's barriers and memory waits
// overlap the other's arithmetic; launched one workgroup per tile.
//
// Decay factors come from block-local cumulative log-decays (log2 units):
// Lam_r = sum_{s=1..r} lambda_{16b+s}, a prefix sum over the 16 lanes of a DPP
// row; P_r = 2^Lam_r and 1/P_r = 2^-Lam_r are within 2^+-108 (normal fp32), and
// the factors across blocks are products of per-block totals, each at most 1.
// Transposes between the row layout and the time-major operands of the W, Ub
// and kg^T products go through MFMA with an identity factor (exact for fp16).
// =============================================================================
template <int D>
struct IntraRB {                                          // D: head size (K = V), 256, 128 or 64
    static constexpr int KS = D / 32;                     // 32-channel k-steps
    static constexpr int AP = 68;                         // sA / sT row pitch (floats)
    static constexpr int TP = 72;                         // KE^T / V^T row pitch (halves)
    static constexpr int NFV = 6;                         // factor vectors per wave
    static constexpr size_t SA = 0;                       // float [64][AP]: A (beta-scaled, strictly lower)
    static constexpr size_t ST = SA + (size_t)64 * AP * 4;     // float [64][AP]: X = (I + A)^-1
    static constexpr size_t SL0 = ST + (size_t)64 * AP * 4;    // float [4][D]: lambda of each block's row 0
    static constexpr size_t SLE = SL0 + 4 * D * 4;             // float [4][D]: Lam at each block's row 15
    static constexpr size_t SBETA = SLE + 4 * D * 4;           // float [64]
    static constexpr size_t SVMAX = SBETA + 64 * 4;            // float [4]
    static constexpr size_t SGB = SVMAX + 64;                  // float [4 waves][D]: gate offsets
    static constexpr size_t U = SGB + 4 * D * 4;               // union of two uses:
    static constexpr size_t FV = U;                            //  per-wave factor vectors [4][NFV][D]
    static constexpr size_t RP = FV + (size_t)4 * NFV * D * 4;     //  R' fragments half8 [3][KS][64]
    static constexpr size_t SX = RP + (size_t)3 * KS * 64 * 16;    //  inverse scratch [4][16][20]
    static constexpr size_t KQ = SX + (size_t)4 * 16 * 20 * 4;     //  KP, QP fragments of block 3, half8 [2][KS][64]
    static constexpr size_t U1_END = KQ + (size_t)2 * KS * 64 * 16;
    static constexpr size_t KET = U;                           //  KE^T fp16 [D][TP] (after the inverse)
    static constexpr size_t VT = KET + (size_t)D * TP * 2;     //  V^T  fp16 [D][TP]
    static constexpr size_t U2_END = VT + (size_t)D * TP * 2;
    static constexpr size_t BYTES = U1_END > U2_END ? U1_END : U2_END;
};

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

template <typename Tin, int D = 128>
__global__ __launch_bounds__(256, D == 256 ? 1 : 2) void intra64_kernel(PrefillArgs p, int64_t ntiles)
{
    constexpr int C = 64, NB = 4, CS = 2;
    constexpr int KS = D / 32, KT = D / 16;   // 32-channel k-steps; 16-channel tiles (= value blocks)
    constexpr int CPL = D / 64;               // channels of a per-channel vector each lane owns
    using R = Record<C, false, D>;
    using LY = IntraRB<D>;
    static_assert(std::is_same<Tin, __bf16>::value, "bf16 inputs");

    __shared__ __align__(16) unsigned char smem[LY::BYTES];
    float (*sA)[LY::AP] = (float (*)[LY::AP])(smem + LY::SA);
    float (*sT)[LY::AP] = (float (*)[LY::AP])(smem + LY::ST);
    float *sL0 = (float *)(smem + LY::SL0);
    float *sLE = (float *)(smem + LY::SLE);
    float *sBeta = (float *)(smem + LY::SBETA);
    float *sVmax = (float *)(smem + LY::SVMAX);
    half8 *sRP = (half8 *)(smem + LY::RP);
    half8 *sKQ = (half8 *)(smem + LY::KQ);
    _Float16 *sKET = (_Float16 *)(smem + LY::KET);
    _Float16 *sVT = (_Float16 *)(smem + LY::VT);

    const int H = p.H;
    const float lb2 = p.lower_bound * kLog2e;

    // blocks (0,1) and (2,3) of T lie above the diagonal but inside the k-steps
    // that the W / Ub products read: zero once (nothing else writes them)
    for (int idx = threadIdx.x; idx < 512; idx += 256) {
        const int blk = idx >> 8, e = idx & 255;
        sT[32 * blk + (e >> 4)][32 * blk + 16 + (e & 15)] = 0.0f;
    }

    // W and Ub results of the previous tile, stored once the next tile's loads are issued
    half8 pw[KS];
    half4_t pu[KT];
    unsigned char *prec = nullptr;
    auto flush = [&](int b, int lane) {
        if (!prec) return;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            *(half8 *)(prec + R::W_OFF + ((size_t)(b * KS + s) * 64 + lane) * 16) = pw[s];
#pragma unroll
        for (int vb = 0; vb < KT; ++vb)
            *(half4_t *)(prec + R::UB_OFF + ((size_t)(vb * NB + b) * 64 + lane) * 8) = pu[vb];
        prec = nullptr;
    };

    for (int64_t ti = blockIdx.x; ti < ntiles; ti += gridDim.x) {
        // lane and wave indices are re-derived every tile (opaque to the
        // compiler), so that the many per-lane addresses below are formed where
        // they are used instead of being hoisted out of the loop into registers
        int tid = threadIdx.x, bw = tid >> 6;
        asm volatile("" : "+v"(tid));
        bw = __builtin_amdgcn_readfirstlane(bw);
        asm volatile("" : "+s"(bw));
        const int b = bw;                           // this wave's 16-row block
        const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
        float *fv = (float *)(smem + LY::FV) + (size_t)b * LY::NFV * D;     // this wave's factor vectors
        // identity selectors: column c of tile 2s + half picks channel tile_chan(2s + half, c),
        // i.e. k-index (c / 4, 4 half + c % 4) of step s
        half8 id0, id1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            id0[e] = (_Float16)((lg == (lr >> 2) && e == (lr & 3)) ? 1.0f : 0.0f);
            id1[e] = (_Float16)((lg == (lr >> 2) && e == 4 + (lr & 3)) ? 1.0f : 0.0f);
        }
        // channel offset of entry (s, half) of this lane: 32 s + 8 lg + 4 half
        auto chan = [&](int s, int hf) { return 32 * s + 8 * lg + 4 * hf; };

        int n = 0, L = 0;
        int64_t t0 = 0;
        // tile = slot * H + head (below 2^31: the launch checks it)
        const uint32_t slot_u = (uint32_t)ti / (uint32_t)H;
        if (!locate_slot<C>(p.cu_seqlens, p.N, (int64_t)slot_u, n, t0, L)) continue;   // unused slot
        const int h = (int)((uint32_t)ti - slot_u * (uint32_t)H);
        unsigned char *rec = p.ws + (size_t)ti * R::BYTES;

        // ---- loads: gates first (consumed first), then q, k, v, beta ----------------
        const int r = 16 * b + lr;                  // tile row of this lane
        const bool rv = r < L;
        const size_t row = (size_t)(t0 + (rv ? r : L - 1)) * H + h;
        const float *gr = p.g + row * D;
        f32x4 graw[KS][2];
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) graw[s][hf] = *(const f32x4 *)(gr + chan(s, hf));
        float dtv[CPL];                              // dt_bias of channels CPL lane .. + CPL - 1
        if constexpr (CPL == 4) {
            const f32x4 d4 = *(const f32x4 *)(p.dt_bias + (size_t)h * D + 4 * lane);
#pragma unroll
            for (int c = 0; c < CPL; ++c) dtv[c] = d4[c];
        } else if constexpr (CPL == 2) {
            const float2 d2 = *(const float2 *)(p.dt_bias + (size_t)h * D + 2 * lane);
            dtv[0] = d2.x;
            dtv[CPL - 1] = d2.y;
        } else {
            dtv[0] = p.dt_bias[(size_t)h * D + lane];
        }
        const size_t rowk = (size_t)(t0 + (rv ? r : L - 1)) * p.Hk + h / (H / p.Hk);
        const Tin *qr = (const Tin *)p.q + rowk * D;
        const Tin *kr = (const Tin *)p.k + rowk * D;
        const Tin *vr = (const Tin *)p.v + row * D;
        bf16x8 qraw[KS], kraw[KS], vraw[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qraw[s] = *(const bf16x8 *)(qr + chan(s, 0));
            kraw[s] = *(const bf16x8 *)(kr + chan(s, 0));
            vraw[s] = *(const bf16x8 *)(vr + chan(s, 0));
        }
        const float braw = p.beta_raw[row];
        const float alog = *(const __attribute__((address_space(4))) float *)(p.A_log + h);


        // ---- gates and block-local cumulative log-decay ------------------------------
        // sigmoid(a (g + db)) = 1 / (1 + 2^(ga g + ga db)), ga = -a log2e; lambda in
        // log2 units = lb2 * sigmoid; rows past the chunk end get lambda = 0
        const float ga = -fast_exp2(alog * kLog2e) * kLog2e;
        // ga * dt_bias per channel, spread to this lane's channels through this
        // wave's own LDS row (its LDS accesses complete in order)
        float *sgb = (float *)(smem + LY::SGB) + b * D;
#pragma unroll
        for (int c = 0; c < CPL; ++c) sgb[CPL * lane + c] = ga * dtv[c];
        float lam[KS][8];
        const float lbr = rv ? lb2 : 0.0f;           // rows past the chunk end: lambda = 0
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const f32x4 gb = *(const f32x4 *)(sgb + chan(s, hf));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float sg = fast_rcp(1.0f + fast_exp2(fmaf(graw[s][hf][i], ga, gb[i])));
                    lam[s][4 * hf + i] = lbr * sg;
                }
            }
        if (lr == 0) {                               // lambda of the block's first row
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    *(f32x4 *)(sL0 + b * D + chan(s, hf)) =
                        f32x4{lam[s][4 * hf], lam[s][4 * hf + 1], lam[s][4 * hf + 2], lam[s][4 * hf + 3]};
        }
        // Lam_r = sum_{s=1..r} lambda_s over the block: inclusive prefix sum across
        // the 16 lanes of the DPP row (row_shr d, out-of-row lanes read 0)
        float Lm[KS][8];
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) Lm[s][e] = (lr == 0) ? 0.0f : lam[s][e];
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) Lm[s][e] += dpp_f<0x111>(Lm[s][e]);
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) Lm[s][e] += dpp_f<0x112>(Lm[s][e]);
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) Lm[s][e] += dpp_f<0x114>(Lm[s][e]);
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) Lm[s][e] += dpp_f<0x118>(Lm[s][e]);
        if (lr == 15) {
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    *(f32x4 *)(sLE + b * D + chan(s, hf)) =
                        f32x4{Lm[s][4 * hf], Lm[s][4 * hf + 1], Lm[s][4 * hf + 2], Lm[s][4 * hf + 3]};
        }
        // largest |v| of the lane on the bf16 bit patterns: with the sign cleared their
        // unsigned order is the numeric order (two 16-bit lanes per instruction)
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        u16x2 vm2 = {0, 0};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
            const u32x4v w = __builtin_bit_cast(u32x4v, vraw[s]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u16x2 x = __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu);
                vm2 = __builtin_elementwise_max(vm2, x);
            }
        }
        float vmax = __uint_as_float((uint32_t)(vm2[0] > vm2[1] ? vm2[0] : vm2[1]) << 16);
        vmax = wave_max_nonneg(vmax);
        if (lane == 0) sVmax[b] = vmax;
        lds_barrier();                                                     // B1
        // the previous tile's W / Ub, now behind this tile's loads in the memory queue
        flush(b, lane);

        // ---- per-channel factors (lane: channels CPL lane .. CPL lane + CPL - 1) --------
        //   QF_b = e^{G_16b}                      (chunk-relative, row 16b included)
        //   KF_b = prod of the block totals after b
        //   Pe_b = 2^Lam_15 of block b
        //   X_bc = e^{G_16b - G_16c+15}, c < b
        // (specialised on the wave's block b, so that its branches are resolved at compile time)
        auto factors = [&](auto bc) {
            constexpr int b = decltype(bc)::value;
            float tot[NB][CPL], l0b[CPL], leb[CPL];
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const float x0 = sL0[bb * D + CPL * lane + c];
                    const float xe = sLE[bb * D + CPL * lane + c];
                    tot[bb][c] = x0 + xe;
                    if (bb == b) { l0b[c] = x0; leb[c] = xe; }
                }
            }
            float qf[CPL], kf[CPL], xs[NB][CPL], all[CPL];
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                float pre = 0.f, suf = 0.f, sum = 0.f;
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) {
                    if (bb < b) pre += tot[bb][i];
                    if (bb > b) suf += tot[bb][i];
                    sum += tot[bb][i];
                }
                qf[i] = pre + l0b[i];
                kf[i] = suf;
                all[i] = sum;
                // X_bc: lambda of row 16b plus the totals of the blocks strictly between
                float run = l0b[i];
#pragma unroll
                for (int c = NB - 1; c >= 0; --c) {
                    if (c < b) {
                        xs[c][i] = run;
                        run += tot[c][i];
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                fv[0 * D + CPL * lane + c] = fast_exp2(qf[c]);
                fv[1 * D + CPL * lane + c] = fast_exp2(kf[c]);
                fv[2 * D + CPL * lane + c] = fast_exp2(leb[c]);
#pragma unroll
                for (int cc = 0; cc < NB - 1; ++cc)
                    if (cc < b) fv[(3 + cc) * D + CPL * lane + c] = fast_exp2(xs[cc][c]);
                if (b == 0)                          // total decay of the chunk
                    ((float *)(rec + R::GC_OFF))[CPL * lane + c] = fast_exp2(all[c]);
            }
        };
        switch (b) {
        case 0: factors(std::integral_constant<int, 0>{}); break;
        case 1: factors(std::integral_constant<int, 1>{}); break;
        case 2: factors(std::integral_constant<int, 2>{}); break;
        default: factors(std::integral_constant<int, 3>{}); break;
        }
        if (lg == 0) sBeta[r] = rv ? sigmoid_f(braw) : 0.0f;
        const float beta = rv ? sigmoid_f(braw) : 0.0f;
        // power-of-two scale of v for the fp16 product T v (exact)
        float vscale, vinv;
        {
            const float m = fmaxf(fmaxf(sVmax[0], sVmax[1]), fmaxf(sVmax[2], sVmax[3]));
            vscale = pow2_scale_for(m, 9);          // |T v / vscale| <= 64 * 2^9 = 2^15
            vinv = inv_pow2(vscale);
            if (tid == 0) *(float *)(rec + R::UBS_OFF) = (m > 0.f) ? vscale : 0.0f;
        }

        // ---- row quantities: norms, decay products, fp16 operands ---------------------
        float KP[KS][8], QP[KS][8], RI[KS][8];
        half8 ke16[KS], v16[KS];
        {
            // sums of squares two channels at a time on the bf16 dot product
            // (exact products, fp32 sums)
            float sq = 0.f, sk = 0.f;
            typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const bf16x2_t q2 = {qraw[s][e], qraw[s][e + 1]}, k2 = {kraw[s][e], kraw[s][e + 1]};
                    sq = __builtin_amdgcn_fdot2_f32_bf16(q2, q2, sq, false);
                    sk = __builtin_amdgcn_fdot2_f32_bf16(k2, k2, sk, false);
                }
            sq += __shfl_xor(sq, 16);
            sq += __shfl_xor(sq, 32);
            sk += __shfl_xor(sk, 16);
            sk += __shfl_xor(sk, 32);
            const float fq = rsqrtf(sq + kL2Eps) * p.scale, fk = rv ? rsqrtf(sk + kL2Eps) : 0.0f;
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = 4 * hf + i;
                        const float ep = fast_exp2(Lm[s][e]), em = fast_exp2(-Lm[s][e]);
                        const float kh = (float)kraw[s][e] * fk;
                        KP[s][e] = kh * ep;                               // kh e^{G_t - G_16b}
                        QP[s][e] = (float)qraw[s][e] * fq * ep;           // qh e^{G_t - G_16b}
                        RI[s][e] = kh * em;                               // kh e^{G_16b - G_t}
                        v16[s][e] = (_Float16)((float)vraw[s][e] * vinv);
                    }
        }
        // qg, kg^T, KE and the R' operands of the off-diagonal blocks
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            float qf[8], kf[8], pe[8];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const f32x4 a = *(const f32x4 *)(fv + 0 * D + chan(s, hf));
                const f32x4 k = *(const f32x4 *)(fv + 1 * D + chan(s, hf));
                const f32x4 e = *(const f32x4 *)(fv + 2 * D + chan(s, hf));
#pragma unroll
                for (int i = 0; i < 4; ++i) { qf[4 * hf + i] = a[i]; kf[4 * hf + i] = k[i]; pe[4 * hf + i] = e[i]; }
            }
            half8 qg, kg, rp;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float rpe = RI[s][e] * pe[e];          // kh e^{G_16b+15 - G_t} <= |kh|
                rp[e] = (_Float16)rpe;
                kg[e] = (_Float16)(rpe * kf[e]);             // kh e^{G_C - G_t}
                qg[e] = (_Float16)(QP[s][e] * qf[e]);        // qh e^{G_t}
                ke16[s][e] = (_Float16)(KP[s][e] * qf[e]);   // kh e^{G_t}
            }
            if (b < NB - 1) sRP[(b * KS + s) * 64 + lane] = rp;
            if (b == NB - 1) {          // left operands of the blocks (3, 0), (3, 1), computed by waves 0, 1
                half8 kq, qq;
#pragma unroll
                for (int e = 0; e < 8; ++e) { kq[e] = (_Float16)KP[s][e]; qq[e] = (_Float16)QP[s][e]; }
                sKQ[s * 64 + lane] = kq;
                sKQ[(KS + s) * 64 + lane] = qq;
            }
            *(half8 *)(rec + R::QG_OFF + ((size_t)(b * KS + s) * 64 + lane) * 16) = qg;
            // kg^T fragments (tile 2s + half, k-step b / 2): this block's rows are
            // positions 4 (b & 1) .. + 3 of each lane's 8
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const f32x4 t = mfma_h(kg, hf ? id1 : id0, f32x4{0.f, 0.f, 0.f, 0.f});
                *(half4_t *)(rec + R::KG_OFF + ((size_t)((2 * s + hf) * CS + (b >> 1)) * 64 + lane) * 16 + 8 * (b & 1)) =
                    half4_t{(_Float16)t[0], (_Float16)t[1], (_Float16)t[2], (_Float16)t[3]};
            }
        }
        lds_barrier();                                                     // B2: R' visible

        // ---- A and M blocks of row block b ------------------------------------------
        // lane holds A[i][j] / M[i][j] for i = 16b + lr, j = 16c + 4lg + ii
        {
            f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {              // diagonal block: fp32 MFMA (factors up to 2^108)
                aA = mfma_f32x8(RI[s], KP[s], aA);
                aM = mfma_f32x8(RI[s], QP[s], aM);
            }
            f32x4 av;
            float xm[8];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int j = 4 * lg + ii;
                av[ii] = (lr > j) ? beta * aA[ii] : 0.0f;
                xm[ii] = (j <= lr) ? aM[ii] : 0.0f;
                xm[ii + 4] = 0.0f;
            }
            *(f32x4 *)&sA[16 * b + lr][16 * b + 4 * lg] = av;
            unsigned char *mf = rec + R::M_OFF + ((size_t)(b * CS + (b >> 1)) * 64 + lane) * 16;
            if ((b & 1) == 0)
                *(half8 *)mf = half8{(_Float16)xm[0], (_Float16)xm[1], (_Float16)xm[2], (_Float16)xm[3],
                                     (_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
            else
                *(half4_t *)(mf + 8) = half4_t{(_Float16)xm[0], (_Float16)xm[1], (_Float16)xm[2], (_Float16)xm[3]};
        }
        // off-diagonal blocks (b, c), c < b, on fp16 MFMA: by the row owner b, except
        // (3, 0) and (3, 1), which the column owners 0 and 1 take (two blocks per
        // wave at most instead of three)
        for (int c = (b == NB - 1 ? 2 : 0); c < b; ++c) {
            f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aM = {0.f, 0.f, 0.f, 0.f};
            const float *xf = fv + (3 + c) * D;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const half8 rpc = sRP[(c * KS + s) * 64 + lane];
                const f32x4 x0 = *(const f32x4 *)(xf + chan(s, 0)), x1 = *(const f32x4 *)(xf + chan(s, 1));
                half8 lk, lq;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    lk[i] = (_Float16)(KP[s][i] * x0[i]);
                    lk[i + 4] = (_Float16)(KP[s][i + 4] * x1[i]);
                    lq[i] = (_Float16)(QP[s][i] * x0[i]);
                    lq[i + 4] = (_Float16)(QP[s][i + 4] * x1[i]);
                }
                aA = mfma_h(rpc, lk, aA);
                aM = mfma_h(rpc, lq, aM);
            }
            *(f32x4 *)&sA[16 * b + lr][16 * c + 4 * lg] = aA * beta;
            *(half4_t *)(rec + R::M_OFF + ((size_t)(b * CS + (c >> 1)) * 64 + lane) * 16 + 8 * (c & 1)) =
                half4_t{(_Float16)aM[0], (_Float16)aM[1], (_Float16)aM[2], (_Float16)aM[3]};
        }
        if (b < 2) {                                    // block (3, b) by its column owner
            constexpr int a = NB - 1;
            f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aM = {0.f, 0.f, 0.f, 0.f};
            const float *xf = (const float *)(smem + LY::FV) + (size_t)a * LY::NFV * D + (3 + b) * D;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const f32x4 x0 = *(const f32x4 *)(xf + chan(s, 0)), x1 = *(const f32x4 *)(xf + chan(s, 1));
                const f32x4 p0 = *(const f32x4 *)(fv + 2 * D + chan(s, 0)), p1 = *(const f32x4 *)(fv + 2 * D + chan(s, 1));
                half8 rr;                                   // kh_j e^{G_48 - G_j}
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    rr[i] = (_Float16)(RI[s][i] * (p0[i] * x0[i]));
                    rr[i + 4] = (_Float16)(RI[s][i + 4] * (p1[i] * x1[i]));
                }
                aA = mfma_h(rr, sKQ[s * 64 + lane], aA);
                aM = mfma_h(rr, sKQ[(KS + s) * 64 + lane], aM);
            }
            // lane holds A[i][j] / M[i][j] for i = 48 + lr, j = 16b + 4lg + ii
            *(f32x4 *)&sA[16 * a + lr][16 * b + 4 * lg] = aA * sBeta[16 * a + lr];
            *(half4_t *)(rec + R::M_OFF + ((size_t)(a * CS + (b >> 1)) * 64 + lane) * 16 + 8 * (b & 1)) =
                half4_t{(_Float16)aM[0], (_Float16)aM[1], (_Float16)aM[2], (_Float16)aM[3]};
        }
        // diagonal block of (I + A)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8) (A^16 = 0);
        // this wave wrote A_bb above and its LDS accesses complete in order
        {
            const float *Ab = &sA[16 * b][16 * b];
            float *Sx = (float *)(smem + LY::SX) + b * 16 * 20;
            const f32x4 p1 = lds_right16(Ab, LY::AP, lr, lg);
            f32x4 z;
#pragma unroll
            for (int i = 0; i < 4; ++i) z[i] = ((4 * lg + i == lr) ? 1.0f : 0.0f) - p1[i];
            f32x4 pw2 = mm16(lds_left16(Ab, LY::AP, lr, lg), p1, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                lds_store16(Sx, 20, pw2, lr, lg);
                const f32x4 lp = lds_left16(Sx, 20, lr, lg);
                z = mm16(lp, z, z);                          // z += A^(2^(m+1)) z
                if (m < 2) pw2 = mm16(lp, pw2, f32x4{0.f, 0.f, 0.f, 0.f});
            }
            lds_store16(&sT[16 * b][16 * b], LY::AP, z, lr, lg);
        }
        lds_barrier();                                                     // B3

        // ---- off-diagonal blocks of X, level 1: X_10, X_32 ----------------------------
        if (b < 2) {
            const int a = 2 * b + 1, c = 2 * b;
            const f32x4 y = mm16(lds_left16(&sA[16 * a][16 * c], LY::AP, lr, lg),
                                 lds_right16(&sT[16 * c][16 * c], LY::AP, lr, lg), f32x4{0.f, 0.f, 0.f, 0.f});
            const f32x4 x = mm16(lds_left16(&sT[16 * a][16 * a], LY::AP, lr, lg), y, f32x4{0.f, 0.f, 0.f, 0.f});
            lds_store16(&sT[16 * a][16 * c], LY::AP, -x, lr, lg);
        }
        // KE^T and V^T (time-major fp16 rows per channel) for the W and Ub products
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int ch = tile_chan(2 * s + hf, lr);
                const f32x4 tk = mfma_h(ke16[s], hf ? id1 : id0, f32x4{0.f, 0.f, 0.f, 0.f});
                const f32x4 tv = mfma_h(v16[s], hf ? id1 : id0, f32x4{0.f, 0.f, 0.f, 0.f});
                *(half4_t *)(sKET + ch * LY::TP + 16 * b + 4 * lg) =
                    half4_t{(_Float16)tk[0], (_Float16)tk[1], (_Float16)tk[2], (_Float16)tk[3]};
                *(half4_t *)(sVT + ch * LY::TP + 16 * b + 4 * lg) =
                    half4_t{(_Float16)tv[0], (_Float16)tv[1], (_Float16)tv[2], (_Float16)tv[3]};
            }
        lds_barrier();                                                     // B4

        // ---- level 2: X_20, X_21, X_30, X_31 (one per wave) ---------------------------
        {
            const int rr = 2 + (b >> 1), c = b & 1;
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            const f32x4 x1c = lds_right16(&sT[16][16 * c], LY::AP, lr, lg);    // X_1c
            f32x4 x00 = zero;
            if (c == 0) x00 = lds_right16(&sT[0][0], LY::AP, lr, lg);
            f32x4 y2 = mm16(lds_left16(&sA[32][16], LY::AP, lr, lg), x1c, zero);            // A_21 X_1c
            if (c == 0) y2 = mm16(lds_left16(&sA[32][0], LY::AP, lr, lg), x00, y2);         // + A_20 X_00
            f32x4 x;
            if (rr == 2) {
                x = mm16(lds_left16(&sT[32][32], LY::AP, lr, lg), y2, zero);                // X_22 Y_2c
            } else {
                f32x4 y3 = mm16(lds_left16(&sA[48][16], LY::AP, lr, lg), x1c, zero);        // A_31 X_1c
                if (c == 0) y3 = mm16(lds_left16(&sA[48][0], LY::AP, lr, lg), x00, y3);     // + A_30 X_00
                x = mm16(lds_left16(&sT[48][32], LY::AP, lr, lg), y2, zero);                // X_32 Y_2c
                x = mm16(lds_left16(&sT[48][48], LY::AP, lr, lg), y3, x);                   // + X_33 Y_3c
            }
            lds_store16(&sT[16 * rr][16 * c], LY::AP, -x, lr, lg);
        }
        lds_barrier();                                                     // B5: T complete

        // ---- W^T = KE^T T^T and Ub = T V for this wave's rows ---------------------------
        {
            const int ns = (b < 2) ? 1 : 2;            // k-steps over t that T's rows reach
            auto t_frag = [&](int tb, int sp) {         // T row fragment, rows of block tb
                float bt[8];
                load_T_row(&sT[16 * tb + lr][32 * sp + 8 * lg], &sBeta[32 * sp + 8 * lg], bt);
                half8 f;
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = (_Float16)bt[e];
                return f;
            };
            half8 tf[CS];
#pragma unroll
            for (int sp = 0; sp < CS; ++sp) {
                if (sp < ns) tf[sp] = t_frag(b, sp);
                else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) tf[sp][e] = (_Float16)0.0f;
                }
            }
            f32x4 aw[KT];
#pragma unroll
            for (int cb = 0; cb < KT; ++cb) {
                aw[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sp = 0; sp < CS; ++sp)
                    if (sp < ns)
                        aw[cb] = mfma_h(*(const half8 *)(sKET + tile_chan(cb, lr) * LY::TP + 32 * sp + 8 * lg), tf[sp], aw[cb]);
            }
#pragma unroll
            for (int s = 0; s < KS; ++s)                // W stored negated: U = Ub + (-W) S^T
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pw[s][i] = (_Float16)(-aw[2 * s][i]);
                    pw[s][i + 4] = (_Float16)(-aw[2 * s + 1][i]);
                }
#pragma unroll
            for (int vb = 0; vb < KT; ++vb) {
                f32x4 au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sp = 0; sp < CS; ++sp)
                    if (sp < ns)
                        au = mfma_h(tf[sp], *(const half8 *)(sVT + (16 * vb + lr) * LY::TP + 32 * sp + 8 * lg), au);
                pu[vb] = half4_t{(_Float16)au[0], (_Float16)au[1], (_Float16)au[2], (_Float16)au[3]};
            }
            prec = rec;
        }
    }
    flush(__builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), threadIdx.x & 63);
}

// ---- launchers ----------------------------------------------------------------

// Device queries and function attributes are settled on the first launch on
// each device and cached, so that later launches (for instance under HIP graph
// capture, after an eager warm-up call) make no runtime call besides the launch.
constexpr int kMaxDevices = 64;

static hipError_t cu_count(int &cus) {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices && (cus = cache[dev].load(std::memory_order_relaxed)) > 0)
        return hipSuccess;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess && dev >= 0 && dev < kMaxDevices) cache[dev].store(cus, std::memory_order_relaxed);
    return e;
}

// One flag word per kernel: bit d set once the dynamic-LDS limit is set on device d.
// Zeroes n 8-byte words (grid-stride).
__global__ __launch_bounds__(256) void zero_words_kernel(uint64_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0;
}

static hipError_t set_lds_limit(const void *fn, int lds, std::atomic<uint64_t> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < kMaxDevices) ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_relaxed);
    return e;
}

template <int C, typename Tin, typename Tout, int D>
static hipError_t launch_prefill_t(const PrefillArgs &a) {
    constexpr bool PRECISE = std::is_same<Tin, float>::value;
    static_assert(D == 128 || (C == 64 && !PRECISE), "head sizes 64 and 256: 64-row chunks of bf16 inputs");
    static_assert(IntraRB<D>::BYTES <= 160 * 1024, "intra-chunk LDS");
    const int64_t slots = num_slots(a.T, a.N, C);
    if ((a.stages & 1) && slots > 0) {
        // workgroups walk the tiles blockIdx.x, blockIdx.x + gridDim.x, ...
        int cus = 0;
        hipError_t e = cu_count(cus);
        if (e != hipSuccess) return e;
        const int64_t ntiles = slots * a.H;
        if constexpr (C == 64 && !PRECISE) {
            // register-blocked kernel, two workgroups per CU at a time: one
            // workgroup per tile (a new one starts wherever one finishes, so
            // the two on a CU drift out of phase; persistent workgroups walking
            // the tiles in step measured 7% slower at T=8192, H=96); the kernel
            // decodes tile indices in 32 bits (a workspace of 2^31 records would
            // be over 100 TB)
            if (ntiles > 0x7fffffff) return hipErrorInvalidValue;
            intra64_kernel<Tin, D><<<(unsigned)ntiles, 256, 0, a.stream>>>(a, ntiles);
        } else {
            // persistent (one per CU): each prefetches its next tile's inputs into LDS
            const int64_t grid = ntiles < (int64_t)cus ? ntiles : (int64_t)cus;
            intra_kernel<C, Tin, PRECISE><<<(unsigned)grid, 64 * kIntraWaves, 0, a.stream>>>(a, ntiles);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int nchains = a.N * a.H;
    if ((a.stages & 2) && nchains > 0) {
        using CFG = InterCfg<C, PRECISE, D>;
        const size_t lds = (size_t)CFG::NBUF * CFG::BUF;
        static std::atomic<uint64_t> lds_set{0};          // one flag word per kernel
        hipError_t e = set_lds_limit((const void *)inter_kernel<C, Tout, PRECISE, D>, (int)lds, lds_set);
        if (e != hipSuccess) return e;
        // one workgroup per 64 state rows of a chain (two at D = 128)
        const unsigned groups = (unsigned)(8 * (D / 64) * ((nchains + 7) / 8));
        if constexpr (C == 64 && !PRECISE && D == 128 && !std::is_same<Tout, _Float16>::value) {
            if (a.z) {                  // the fused output epilogue
                constexpr size_t lds_g = CFG::NBUF * CFG::BUF + (2 * 64 * 16 + 2 * 64) * sizeof(float) + 2 * 8192;
                static_assert(lds_g <= 160 * 1024, "LDS");
                static std::atomic<uint64_t> lds_g_set{0};
                e = set_lds_limit((const void *)inter_kernel<C, Tout, PRECISE, D, true>, (int)lds_g, lds_g_set);
                if (e != hipSuccess) return e;
                const size_t words = (size_t)num_slots(a.T, a.N, C) * a.H * 128;
                zero_words_kernel<<<(unsigned)((words + 255) / 256 < 4096 ? (words + 255) / 256 : 4096), 256, 0,
                                    a.stream>>>(a.xchg, words);
                inter_kernel<C, Tout, PRECISE, D, true><<<groups, 320, lds_g, a.stream>>>(a, nchains);
                return hipGetLastError();
            }
        }
        if (a.z) return hipErrorInvalidValue;
        inter_kernel<C, Tout, PRECISE, D><<<groups, 256, lds, a.stream>>>(a, nchains);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <int C>
static hipError_t launch_prefill_c(const PrefillArgs &a) {
    if (a.o_scale) {                    // fp16 outputs with block scales: 64-row chunks, bf16 inputs
        if constexpr (C == 64) {
            if (a.in_bf16) return launch_prefill_t<C, __bf16, _Float16, 128>(a);
        }
        return hipErrorInvalidValue;
    }
    if (a.in_bf16)
        return a.out_bf16 ? launch_prefill_t<C, __bf16, __bf16, 128>(a)
                          : launch_prefill_t<C, __bf16, float, 128>(a);
    return a.out_bf16 ? launch_prefill_t<C, float, __bf16, 128>(a) : launch_prefill_t<C, float, float, 128>(a);
}

// Whether kda_chunk_fwd's inter-chunk kernel can apply the output epilogue
// itself: 64-row chunks of bf16 inputs at D = 128, and every workgroup of the
// launch resident at once (one per CU: the two workgroups of a chain wait on
// each other).
hipError_t prefill_gate_fusable(const PrefillArgs &a, bool &fusable) {
    fusable = false;
    if (a.D != 128 || a.chunk != 64 || !a.in_bf16 || a.stages != 3) return hipSuccess;
    int cus = 0;
    const hipError_t e = cu_count(cus);
    if (e != hipSuccess) return e;
    const int64_t nchains = (int64_t)a.N * a.H;
    fusable = 16 * ((nchains + 7) / 8) <= (int64_t)cus;
    return hipSuccess;
}

hipError_t launch_prefill(const PrefillArgs &args) {
    PrefillArgs a = args;
    if (a.Hk <= 0) a.Hk = a.H;          // no grouping: one q/k head per value head
    if (a.D == 64) {                    // natively sized kernels: 64-row chunks, bf16 inputs
        if (a.chunk != 64 || !a.in_bf16 || a.o_scale) return hipErrorInvalidValue;
        return a.out_bf16 ? launch_prefill_t<64, __bf16, __bf16, 64>(a)
                          : launch_prefill_t<64, __bf16, float, 64>(a);
    }
    if (a.D == 256) {                   // natively sized kernels: 64-row chunks, bf16 inputs
        if (a.chunk != 64 || !a.in_bf16 || a.o_scale || a.z) return hipErrorInvalidValue;
        return a.out_bf16 ? launch_prefill_t<64, __bf16, __bf16, 256>(a)
                          : launch_prefill_t<64, __bf16, float, 256>(a);
    }
    if (a.D != 128) return hipErrorInvalidValue;
    switch (a.chunk) {
        case 16: return launch_prefill_c<16>(a);
        case 32: return launch_prefill_c<32>(a);
        case 64: return launch_prefill_c<64>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
