// Front end of the attention block (kimi_k3 FusedKDAChunkwise page, "CUDA-only
// forward and causal preprocessing"): every channel of the q, k or v
// projection is filtered along time by its own short causal kernel of W taps
// (left padding of W - 1), then passed through SiLU:
//
//   y[t, c] = silu( sum_{i < W} w[c, i] * x[t - (W - 1) + i, c] ),   silu(u) = u sigmoid(u)
//
// Packed sequences restart the history at their first token: the W - 1
// positions before it come from the sequence's carried-in conv state (its last
// W - 1 inputs so far, oldest first), or are zero without one.
//
// Layout: x rows of `channels` elements with row stride x_stride (a q, k or v
// slice of a fused projection can be passed as it is), y [T, channels]
// contiguous, weights [channels, W] fp32, conv states [N, W - 1, channels] in
// x's dtype.
//
// Work split (short_conv_kernel): a thread owns 8 consecutive channels of a
// strip of S tokens; it loads the strip's S rows plus the W - 1 rows before it
// into registers (16- or 32-byte loads, consecutive lanes on consecutive
// channels) and slides the W-row window down the strip, so every input row is
// read once per strip, converted to fp32 once, and every output row written
// once, with non-temporal stores (no access of this kernel reads y, and the
// stores then leave the inputs' lines in the caches). HBM-bound. Strips of one channel block follow each other on one XCD
// (blocks are dealt to the 8 XCDs round-robin), so the W - 1 halo rows of a
// strip were fetched into that XCD's L2 by the strip before it. The few strips
// that touch a sequence start (or the end of the input) take a general path
// (chosen per strip, uniform over the workgroup) that gathers each token's
// window row by row, with the taps before the start read from the conv state.
//
// Final conv states (each sequence's last W - 1 inputs, reaching back into the
// carried-in state for sequences shorter than W - 1) are written by the thread
// that handles the sequence's last token, from its window; empty sequences are
// passed on by the strip that owns their start offset. When the final state
// replaces the carried-in state in place, strips could overwrite a state that
// another strip still has to read, so final_state_kernel writes them instead,
// after short_conv_kernel on the same stream, each thread reading all it needs
// before writing.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kConvThreads = 256;
constexpr int kConvChanPerBlock = 8 * kConvThreads;

template <typename T> struct ConvStrip;
template <> struct ConvStrip<__bf16> { static constexpr int S = 16; };
template <> struct ConvStrip<float> { static constexpr int S = 16; };

// Sequence of token t: the n in [0, N) with cu[n] <= t < cu[n + 1] (empty
// sequences are skipped). Wave-uniform arguments; needs 0 <= t < cu[N].
__device__ __forceinline__ int seq_of(const int64_t *cu, int N, int64_t t) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Logical work item of physical block b. Blocks are dealt to the 8 XCDs
// round-robin (b mod 8); XCD x is given the contiguous logical range
// [x * per, (x + 1) * per), walked in order, where logical ids run over
// strips fastest: consecutive strips of a channel block share an L2.
__device__ __forceinline__ int64_t xcd_logical(int64_t b, int64_t per) {
    return (b & 7) * per + (b >> 3);
}

// silu(u) = u / (1 + e^-u): exp2 of -u log2(e), then the reciprocal. For very
// negative u the exponential overflows to +inf and the reciprocal to 0, which
// is the limit, so no range split is needed.
__device__ __forceinline__ float silu_f(float u) {
    return u * fast_rcp(1.0f + fast_exp2(-u * kLog2e));
}

template <int W>
__device__ __forceinline__ void conv_silu_store_prep(const float (&wt)[W][8], const float (&win)[W][8],
                                                     float (&out)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float acc = wt[W - 1][e] * win[W - 1][e];
#pragma unroll
        for (int i = 0; i < W - 1; ++i) acc = fmaf(wt[i][e], win[i][e], acc);
        out[e] = silu_f(acc);
    }
}

// Final conv state of an empty sequence m: its carried-in state, or zeros.
template <typename T, int W>
__device__ __forceinline__ void pass_state_on_w(const T *st_in, T *st_out, int m, int64_t channels,
                                                int64_t c) {
#pragma unroll
    for (int r = 0; r < W - 1; ++r) {
        const int64_t off = ((int64_t)m * (W - 1) + r) * channels + c;
        Vec8<T> v;
        if (st_in) v.load(st_in + off); else v.zero();
        v.store(st_out + off);
    }
}

template <typename T, int W>
__global__ __launch_bounds__(kConvThreads) void short_conv_kernel(
    const T *__restrict__ x, int64_t x_stride, const float *__restrict__ w,
    const int64_t *__restrict__ cu, int N, int64_t T_total, int64_t channels,
    int64_t nstrips, int64_t per_xcd, int64_t nlogical,
    const T *__restrict__ st_in, T *__restrict__ st_out, T *__restrict__ y,
    const int32_t *__restrict__ slots, int num_slots)
{
    constexpr int S = ConvStrip<T>::S;
    const int64_t L = xcd_logical(blockIdx.x, per_xcd);
    if (L >= nlogical) return;
    const int64_t cb = L / nstrips;
    const int64_t strip = L - cb * nstrips;
    const int64_t c = cb * kConvChanPerBlock + 8 * (int64_t)threadIdx.x;
    if (c >= channels) return;                       // channels % 8 == 0: whole groups
    const int64_t t0 = strip * S;

    float wt[W][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int i = 0; i < W; ++i) wt[i][e] = w[(c + e) * W + i];
    }

    int n = seq_of(cu, N, t0);
    int64_t s0 = cu[n], s1 = cu[n + 1];

    // with a state pool, sequence n's conv state is pool entry slots[n]; an
    // entry outside [0, num_slots) marks a padding sequence (zero outputs, no
    // state read)
    auto state_row = [&](int m) -> int64_t { return slots ? (int64_t)slots[m] : (int64_t)m; };
    auto padding = [&](int m) -> bool {
        return slots && (slots[m] < 0 || slots[m] >= num_slots);
    };

    if (t0 + S < T_total && t0 - s0 >= W - 1 && t0 + S <= s1) {
        if (padding(n)) {
            const float zero[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < S; ++j) store8<T>(y + (t0 + j) * channels + c, zero);
            return;
        }
        // Every window of the strip lies inside one sequence: a plain sliding
        // window. Rows t0 - (W - 1) .. t0 + S - 1 are loaded up front (kept
        // packed) and each is converted to fp32 once, as it enters the window.
        Vec8<T> xr[S + W - 1];
#pragma unroll
        for (int r = 0; r < S + W - 1; ++r) xr[r].load(x + (t0 - (W - 1) + r) * x_stride + c);
        // keep every load of the strip ahead of the arithmetic: left to itself
        // the scheduler sinks them next to their uses to save registers, which
        // exposes one memory latency per token
        __builtin_amdgcn_sched_barrier(0);
        float win[W][8];
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
#pragma unroll
            for (int e = 0; e < 8; ++e) win[i][e] = xr[i][e];
        }
#pragma unroll
        for (int j = 0; j < S; ++j) {
#pragma unroll
            for (int e = 0; e < 8; ++e) win[W - 1][e] = xr[j + W - 1][e];
            float out[8];
            conv_silu_store_prep<W>(wt, win, out);
            store8_nt<T>(y + (t0 + j) * channels + c, out);
#pragma unroll
            for (int i = 0; i < W - 1; ++i) {
#pragma unroll
                for (int e = 0; e < 8; ++e) win[i][e] = win[i + 1][e];
            }
        }
        // the strip ends its sequence: the final conv state is its last W - 1 rows
        if (st_out && t0 + S == s1) {
#pragma unroll
            for (int r = 0; r < W - 1; ++r) xr[S + r].store(st_out + ((int64_t)n * (W - 1) + r) * channels + c);
        }
        return;
    }

    // General strip (a sequence starts within W - 1 rows before or inside it,
    // or it is the last, partial strip): the strip's rows are still loaded up
    // front (rows outside [0, T) read as zero and are never used), and each
    // token assembles its window tap by tap; positions before its sequence's
    // start read the conv state row (p - s0 + W - 1) of that sequence, or zero.
    Vec8<T> xr[S + W - 1];
#pragma unroll
    for (int r = 0; r < S + W - 1; ++r) {
        const int64_t t = t0 - (W - 1) + r;
        if (t >= 0 && t < T_total) xr[r].load(x + t * x_stride + c);
        else xr[r].zero();
    }
    if (st_out) {
        // empty sequences that start at t0 lie before n (the search skips them)
        for (int m = n - 1; m >= 0 && cu[m] == t0; --m) pass_state_on_w<T, W>(st_in, st_out, m, channels, c);
    }
#pragma unroll
    for (int j = 0; j < S; ++j) {
        const int64_t t = t0 + j;
        if (t >= T_total) break;
        while (t >= s1) {
            ++n; s0 = s1; s1 = cu[n + 1];
            if (st_out && s1 == s0) pass_state_on_w<T, W>(st_in, st_out, n, channels, c);   // empty
        }
        if (padding(n)) {
            const float zero[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            store8<T>(y + t * channels + c, zero);
            continue;
        }
        float win[W][8];
#pragma unroll
        for (int i = 0; i < W; ++i) {
            const int64_t p = t - (W - 1) + i;
            if (p >= s0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) win[i][e] = xr[j + i][e];
            } else if (st_in) {
                load8(st_in + (state_row(n) * (W - 1) + (p - s0 + W - 1)) * channels + c, win[i]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) win[i][e] = 0.f;
            }
        }
        float out[8];
        conv_silu_store_prep<W>(wt, win, out);
        store8_nt<T>(y + t * channels + c, out);
        if (st_out && t == s1 - 1) {
            // last token of its sequence: the final conv state is the window's
            // last W - 1 rows (reaching into the carried-in state if short)
#pragma unroll
            for (int r = 0; r < W - 1; ++r) store8<T>(st_out + ((int64_t)n * (W - 1) + r) * channels + c, win[r + 1]);
        }
    }
    if (st_out && t0 + S >= T_total) {
        // the last strip: sequences after the last token's one are empty
        for (int m = n + 1; m < N; ++m) pass_state_on_w<T, W>(st_in, st_out, m, channels, c);
    }
}

// One thread per (sequence, 8 channels): final state row r of sequence n is
// input position len - (W - 1) + r of the sequence, taken from the carried-in
// state (or zero) when that position is negative.
template <typename T, int W>
__global__ __launch_bounds__(kConvThreads) void final_state_kernel(
    const T *__restrict__ x, int64_t x_stride, const int64_t *__restrict__ cu, int N,
    int64_t channels, int64_t ncb, const T *st_in, T *st_out, const int32_t *slots,
    int num_slots)
{
    const int64_t n = blockIdx.x / ncb;
    const int64_t cb = blockIdx.x - n * ncb;
    const int64_t c = cb * kConvChanPerBlock + 8 * (int64_t)threadIdx.x;
    if (n >= N || c >= channels) return;
    int64_t srow = n;                                 // state row: n, or its pool entry
    if (slots) {
        srow = slots[n];
        if (srow < 0 || srow >= num_slots) return;    // padding: no state touched
    }
    const int64_t s0 = cu[n], len = cu[n + 1] - s0;
    float rows[W - 1][8];
#pragma unroll
    for (int r = 0; r < W - 1; ++r) {
        const int64_t p = len - (W - 1) + r;
        if (p >= 0) {
            load8(x + (s0 + p) * x_stride + c, rows[r]);
        } else if (st_in) {
            load8(st_in + (srow * (W - 1) + (W - 1) + p) * channels + c, rows[r]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) rows[r][e] = 0.f;
        }
    }
#pragma unroll
    for (int r = 0; r < W - 1; ++r) store8<T>(st_out + (srow * (W - 1) + r) * channels + c, rows[r]);
}

template <typename T, int W>
hipError_t launch_conv_w(const ShortConvArgs &a) {
    constexpr int S = ConvStrip<T>::S;
    const int64_t ncb = (a.channels + kConvChanPerBlock - 1) / kConvChanPerBlock;
    // the final conv state is written by the conv kernel itself unless it
    // replaces the carried-in state in place (other strips may still read
    // that) or there are no tokens: then a second kernel writes it afterwards
    const bool fused_state = W > 1 && a.st_out && a.st_out != a.st_in && a.T > 0 && !a.slots;
    if (a.T > 0) {
        const int64_t nstrips = (a.T + S - 1) / S;
        const int64_t nlogical = nstrips * ncb;
        const int64_t per = (nlogical + 7) / 8;
        short_conv_kernel<T, W><<<(unsigned)(8 * per), kConvThreads, 0, a.stream>>>(
            (const T *)a.x, a.x_stride, a.w, a.cu, a.N, a.T, a.channels, nstrips, per, nlogical,
            (const T *)a.st_in, fused_state ? (T *)a.st_out : nullptr, (T *)a.y, a.slots,
            a.num_slots);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if constexpr (W > 1) {
        if (a.st_out && !fused_state) {
            final_state_kernel<T, W><<<(unsigned)(a.N * ncb), kConvThreads, 0, a.stream>>>(
                (const T *)a.x, a.x_stride, a.cu, a.N, a.channels, ncb, (const T *)a.st_in,
                (T *)a.st_out, a.slots, a.num_slots);
            return hipGetLastError();
        }
    }
    return hipSuccess;
}

template <typename T>
hipError_t launch_conv_t(const ShortConvArgs &a) {
    switch (a.W) {
        case 1: return launch_conv_w<T, 1>(a);
        case 2: return launch_conv_w<T, 2>(a);
        case 3: return launch_conv_w<T, 3>(a);
        case 4: return launch_conv_w<T, 4>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int64_t short_conv_blocks(int64_t T, int64_t channels, bool bf16) {
    const int S = bf16 ? ConvStrip<__bf16>::S : ConvStrip<float>::S;
    const int64_t ncb = (channels + kConvChanPerBlock - 1) / kConvChanPerBlock;
    return 8 * ((((T + S - 1) / S) * ncb + 7) / 8);
}

int64_t short_conv_state_blocks(int64_t N, int64_t channels) {
    return N * ((channels + kConvChanPerBlock - 1) / kConvChanPerBlock);
}

hipError_t launch_short_conv(const ShortConvArgs &a) {
    return a.bf16 ? launch_conv_t<__bf16>(a) : launch_conv_t<float>(a);
}

}  // namespace kda
