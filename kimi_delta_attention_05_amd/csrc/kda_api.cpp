// libkda C ABI: argument validation (host only, before any HIP call),
// workspace sizing and kernel launches. See include/kda.h for the contract.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <initializer_list>
#include <utility>
#include <string>
#include <vector>

#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

kda_status_t fail(kda_status_t st, const std::string &msg) {
    g_last_error = msg;
    return st;
}

kda_status_t ok() {
    g_last_error.clear();
    return KDA_OK;
}

bool valid_dtype(kda_dtype_t d) { return d == KDA_F32 || d == KDA_BF16; }

// Checks shared by both entry points. Returns KDA_OK or an error with detail.
kda_status_t check_common(int64_t H, int32_t K, int32_t V, float scale, float lower_bound,
                          kda_dtype_t in_dtype, kda_dtype_t o_dtype, bool below_128 = false) {
    if (H < 1 || H > 65536) return fail(KDA_ERR_INVALID_ARG, "H must lie in [1, 65536]");
    if (below_128 ? (K < 1 || K > 128 || V < 1 || V > 128) : (K != 128 || V != 128))
        return fail(KDA_ERR_UNSUPPORTED,
                    std::string(below_128 ? "K and V must lie in [1, 128]" : "only K = V = 128 is supported") +
                        " (got K=" + std::to_string(K) + ", V=" + std::to_string(V) +
                        "; kda_recurrent_fwd takes any K, V up to 256)");
    if (!(scale > 0.0f) || !std::isfinite(scale))
        return fail(KDA_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (!(lower_bound >= -5.0f && lower_bound < 0.0f))
        return fail(KDA_ERR_INVALID_ARG, "lower_bound must lie in [-5, 0)");
    if (!valid_dtype(in_dtype)) return fail(KDA_ERR_UNSUPPORTED, "unknown input dtype");
    if (!valid_dtype(o_dtype)) return fail(KDA_ERR_UNSUPPORTED, "unknown output dtype");
    return KDA_OK;
}

// Vector loads and stores and the global->LDS copies move 16 bytes per lane,
// so every tensor pointer except the scalar per-token/per-head arrays
// (beta_raw, A_log) must be 16-byte aligned. NULL passes.
kda_status_t check_aligned16(std::initializer_list<std::pair<const void *, const char *>> ptrs) {
    for (const auto &pn : ptrs)
        if (((uintptr_t)pn.first & 15) != 0)
            return fail(KDA_ERR_INVALID_ARG, std::string(pn.second) + " must be 16-byte aligned");
    return KDA_OK;
}

// Byte ranges of caller buffers, for the checks that outputs do not overlap
// inputs other threads still read. A NULL pointer or zero size is empty.
struct ByteRange {
    uintptr_t lo = 0, hi = 0;
};
ByteRange byte_range(const void *p, uintptr_t bytes) {
    return p && bytes ? ByteRange{(uintptr_t)p, (uintptr_t)p + bytes} : ByteRange{};
}
bool overlaps(ByteRange a, ByteRange b) { return a.lo < b.hi && b.lo < a.hi; }

// Argument checks shared by the two front-end entry points.
kda_status_t check_short_conv(const void *x, int64_t x_stride, const float *weight, int32_t W,
                              const int64_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                              int64_t channels, kda_dtype_t dtype, const void *y) {
    if (num_seqs < 1) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 1");
    if (total_tokens < 0) return fail(KDA_ERR_INVALID_ARG, "total_tokens must be >= 0");
    if (W < 1 || W > 4)
        return fail(KDA_ERR_UNSUPPORTED, "kernel size W must lie in [1, 4] (got " + std::to_string(W) + ")");
    if (channels < 8 || channels % 8 != 0)
        return fail(KDA_ERR_INVALID_ARG, "channels must be a positive multiple of 8");
    if (x_stride < channels || x_stride % 8 != 0)
        return fail(KDA_ERR_INVALID_ARG, "x_stride must be a multiple of 8 and >= channels");
    if (!valid_dtype(dtype)) return fail(KDA_ERR_UNSUPPORTED, "unknown dtype");
    if (!cu_seqlens || !weight) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens and weight must not be NULL");
    if (total_tokens > 0 && (!x || !y)) return fail(KDA_ERR_INVALID_ARG, "x and y must not be NULL");
    if (((uintptr_t)weight & 3) != 0 || ((uintptr_t)cu_seqlens & 7) != 0)
        return fail(KDA_ERR_INVALID_ARG, "weight must be 4-byte and cu_seqlens 8-byte aligned");
    if (kda::short_conv_blocks(total_tokens, channels, dtype == KDA_BF16) > (int64_t)0x7fffffff ||
        kda::short_conv_state_blocks(num_seqs, channels) > (int64_t)0x7fffffff)
        return fail(KDA_ERR_INVALID_ARG, "total_tokens * channels too large for one launch");
    return KDA_OK;
}

// Grouped value heads: H value heads share H_qk q/k heads, H a multiple of H_qk.
kda_status_t check_groups(int64_t H, int64_t H_qk) {
    if (H_qk < 1 || H_qk > H || H % H_qk != 0)
        return fail(KDA_ERR_INVALID_ARG, "H_qk must divide H (got H=" + std::to_string(H) +
                                             ", H_qk=" + std::to_string(H_qk) + ")");
    return KDA_OK;
}

kda_status_t hip_fail(hipError_t e, const char *where) {
    return fail(KDA_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

// The head size the chunkwise kernels run at directly: 128, and 64 or 256 for
// K = V = 64 or 256 with 64-row chunks of bf16 inputs (kernels sized for them);
// 0 when the inputs are zero-padded to 128 instead.
int native_head_size(int32_t K, int32_t V, int32_t chunk_size, kda_dtype_t in_dtype) {
    if (K == 128 && V == 128) return 128;
    if (K == V && (K == 64 || K == 256) && chunk_size == 64 && in_dtype == KDA_BF16) return K;
    return 0;
}

// Other head sizes run on the chunkwise kernels over copies of the inputs padded
// with zeros to D key channels and D value rows, D = 128 when K, V <= 128 and
// D = 256 above (64-row chunks of bf16 inputs only), kept in the workspace
// after the per-chunk records: padded key channels have k = q = 0 and padded
// value rows v = 0 and a zero initial state, so they stay exactly zero through
// the recurrence and change neither the norms nor any dot product of the real
// channels; the outputs and final states are the real rows and channels of the
// padded results. 0: no chunkwise form for these sizes.
int padded_head_size(int32_t K, int32_t V, int32_t chunk_size, kda_dtype_t in_dtype) {
    if (K < 1 || V < 1 || K > 256 || V > 256) return 0;
    if (K <= 128 && V <= 128) return 128;
    return (chunk_size == 64 && in_dtype == KDA_BF16) ? 256 : 0;
}
struct PadLayout {
    size_t q, k, v, g, dtb, state, o, end;
};
PadLayout pad_layout(int64_t T, int64_t N, int64_t H, kda_dtype_t in_dtype, size_t base,
                     size_t D) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t esz = in_dtype == KDA_BF16 ? 2 : 4;
    PadLayout L;
    L.q = up(base);
    L.k = up(L.q + (size_t)T * H * D * esz);
    L.v = up(L.k + (size_t)T * H * D * esz);
    L.g = up(L.v + (size_t)T * H * D * esz);
    L.dtb = up(L.g + (size_t)T * H * D * 4);
    L.state = up(L.dtb + (size_t)H * D * 4);
    L.o = up(L.state + (size_t)N * H * D * D * 4);
    L.end = up(L.o + (size_t)T * H * D * 4);
    return L;
}

// The backward's padded copies (head sizes below 128), after its own layout:
// the inputs and adjoints widened to 128, and the gradients at 128 before they
// are narrowed back into the caller's buffers.
struct BwdPadLayout {
    size_t q, k, v, g, dtb, h0, dout, dht, dq, dk, dv, dg, ddt, dh0, end;
};
BwdPadLayout bwd_pad_layout(int64_t T, int64_t N, int64_t H, size_t base) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t D = kda::kHeadDimHost, tok = (size_t)T * H * D * 4, st = (size_t)N * H * D * D * 4;
    BwdPadLayout L;
    L.q = up(base);
    L.k = up(L.q + tok);
    L.v = up(L.k + tok);
    L.g = up(L.v + tok);
    L.dtb = up(L.g + tok);
    L.h0 = up(L.dtb + (size_t)H * D * 4);
    L.dout = up(L.h0 + st);
    L.dht = up(L.dout + tok);
    L.dq = up(L.dht + st);
    L.dk = up(L.dq + tok);
    L.dv = up(L.dk + tok);
    L.dg = up(L.dv + tok);
    L.ddt = up(L.dg + tok);
    L.dh0 = up(L.ddt + (size_t)H * D * 4);
    L.end = up(L.dh0 + st);
    return L;
}

// The decode step with an optional fused output epilogue (z == NULL: none).
kda_status_t decode_step_impl(const void *q, const void *k, const void *v,
                              const float *g, const float *beta_raw,
                              const float *A_log, const float *dt_bias,
                              float scale, float lower_bound,
                              float *state, void *o, kda_dtype_t o_dtype,
                              int32_t B, int32_t H, int32_t K, int32_t V,
                              kda_dtype_t in_dtype, void *stream,
                              const void *z, const float *norm_weight, float norm_eps,
                              const int32_t *slots, int32_t num_slots,
                              const char *name, int32_t H_qk) {
    if (B < 1) return fail(KDA_ERR_INVALID_ARG, "B must be >= 1");
    const bool general = (K != 128 || V != 128) && K >= 1 && K <= 256 && V >= 1 && V <= 256;
    kda_status_t st = check_common(H, general ? 128 : K, general ? 128 : V, scale, lower_bound,
                                   in_dtype, o_dtype);
    if (st != KDA_OK) return st;
    st = check_groups(H, H_qk);
    if (st != KDA_OK) return st;
    if (!q || !k || !v || !g || !beta_raw || !A_log || !dt_bias || !state || !o)
        return fail(KDA_ERR_INVALID_ARG, "a required pointer is NULL");
    if ((int64_t)B * H * 2 > ((int64_t)1 << 31) - 1)     // two workgroups per (request, head)
        return fail(KDA_ERR_INVALID_ARG, "B * H too large");
    st = check_aligned16({{q, "q"}, {k, "k"}, {v, "v"}, {g, "g"}, {dt_bias, "dt_bias"},
                          {state, "state"}, {o, "o"}});
    if (st != KDA_OK) return st;
    if (((uintptr_t)beta_raw & 3) != 0 || ((uintptr_t)A_log & 3) != 0)
        return fail(KDA_ERR_INVALID_ARG, "beta_raw and A_log must be 4-byte aligned");

    if (z) {
        if (!norm_weight) return fail(KDA_ERR_INVALID_ARG, "norm_weight is NULL");
        if (!(norm_eps > 0.0f) || !std::isfinite(norm_eps))
            return fail(KDA_ERR_INVALID_ARG, "norm_eps must be finite and > 0");
        st = check_aligned16({{z, "z"}, {norm_weight, "norm_weight"}});
        if (st != KDA_OK) return st;
    }

    if (general) {
        // other head sizes: the token-by-token kernel with one token per request
        // (no offsets: request n is sequence n), the state updated in place
        if (kda::general_blocks(B, H, V) > (int64_t)0x7fffffff)
            return fail(KDA_ERR_INVALID_ARG, "B * H * V too large for one launch");
        kda::GeneralArgs ga;
        ga.q = q; ga.k = k; ga.v = v; ga.g = g; ga.beta_raw = beta_raw; ga.A_log = A_log;
        ga.dt_bias = dt_bias; ga.scale = scale; ga.lower_bound = lower_bound;
        ga.cu_seqlens = nullptr; ga.N = B; ga.H = H; ga.Hk = H_qk; ga.K = K; ga.V = V;
        ga.h0 = state; ga.ht = state; ga.o = o;
        ga.in_bf16 = in_dtype == KDA_BF16; ga.out_bf16 = o_dtype == KDA_BF16;
        ga.stream = (hipStream_t)stream;
        ga.slots = slots; ga.num_slots = num_slots;
        hipError_t e = kda::launch_recurrent_fwd(ga);
        if (e == hipSuccess && z) {
            // the output epilogue over each (request, head) row of V outputs, in
            // place: the row spans several of the step's workgroups, so it runs
            // as a second pass (padding requests' zero rows stay zero)
            kda::NormGateArgs na;
            na.o = o; na.z = z; na.w = norm_weight; na.eps = norm_eps; na.rows = (int64_t)B * H;
            na.D = V; na.bf16 = o_dtype == KDA_BF16; na.z_bf16 = in_dtype == KDA_BF16;
            na.y_bf16 = na.bf16; na.y = o;
            na.stream = (hipStream_t)stream;
            e = kda::launch_norm_gate(na);
        }
        if (e != hipSuccess) return hip_fail(e, name);
        return ok();
    }

    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta_raw = beta_raw; a.A_log = A_log; a.dt_bias = dt_bias;
    a.scale = scale; a.lower_bound = lower_bound; a.state = state; a.o = o;
    a.B = B; a.H = H; a.in_bf16 = in_dtype == KDA_BF16; a.out_bf16 = o_dtype == KDA_BF16;
    a.stream = (hipStream_t)stream;
    a.z = z; a.norm_w = norm_weight; a.norm_eps = norm_eps;
    a.slots = slots; a.num_slots = num_slots; a.Hk = H_qk;
    hipError_t e = kda::launch_decode(a);
    if (e != hipSuccess) return hip_fail(e, name);
    return ok();
}

}  // namespace

extern "C" {

int kda_version(void) { return 106; }

const char *kda_status_string(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARG: return "invalid argument";
        case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
        case KDA_ERR_WORKSPACE: return "workspace missing or too small";
        case KDA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *kda_last_error(void) { return g_last_error.c_str(); }

size_t kda_chunk_fwd_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                    int32_t K, int32_t V, int32_t chunk_size,
                                    kda_dtype_t in_dtype) {
    if (total_tokens < 0 || num_seqs < 1 || H < 1 || H > 65536) {
        fail(KDA_ERR_INVALID_ARG, "need total_tokens >= 0, num_seqs >= 1, 1 <= H <= 65536");
        return 0;
    }
    if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) {
        fail(KDA_ERR_UNSUPPORTED, "chunk_size must be 16, 32 or 64");
        return 0;
    }
    if (!valid_dtype(in_dtype)) { fail(KDA_ERR_UNSUPPORTED, "unknown input dtype"); return 0; }
    const int native = native_head_size(K, V, chunk_size, in_dtype);
    const int D = native ? native : padded_head_size(K, V, chunk_size, in_dtype);
    if (D == 0) {
        fail(KDA_ERR_UNSUPPORTED, "K and V must lie in [1, 128], or in [1, 256] with chunk_size 64 "
                                  "and bf16 inputs");
        return 0;
    }
    const int64_t slots = kda::num_slots(total_tokens, num_seqs, chunk_size);
    g_last_error.clear();
    // records sized for the head size the kernels run at (64 and 256: 64-row
    // chunks of bf16 inputs)
    const size_t rec = D == 128 ? kda::record_bytes(chunk_size, in_dtype == KDA_F32)
                                : kda::record_bytes(64, false, D);
    const size_t base = (size_t)slots * (size_t)H * rec + 256;
    if (native) return base;
    return pad_layout(total_tokens, num_seqs, H, in_dtype, base, (size_t)D).end;
}

size_t kda_chunk_fwd_gated_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                          int32_t K, int32_t V, int32_t chunk_size,
                                          kda_dtype_t in_dtype, kda_dtype_t o_dtype) {
    const size_t base = kda_chunk_fwd_workspace_size(total_tokens, num_seqs, H, K, V, chunk_size,
                                                     in_dtype);
    if (base == 0) return 0;
    if (!valid_dtype(o_dtype)) { fail(KDA_ERR_UNSUPPORTED, "unknown output dtype"); return 0; }
    const size_t rows = (size_t)total_tokens * H;
    size_t extra = 0;
    if (native_head_size(K, V, chunk_size, in_dtype) == 128 && chunk_size == 64 &&
        in_dtype == KDA_BF16) {
        // the epilogue fused in the inter-chunk kernel: its row-sum exchange; when
        // the batch has too many sequences for that, bf16 results are staged in
        // fp16 with a power-of-two scale per 16 features
        const size_t xchg = (size_t)kda::num_slots(total_tokens, num_seqs, 64) * H * 128 * 8;
        const size_t staged = o_dtype == KDA_BF16 ? rows * V * 2 + rows * (V / 16) * 4 : 0;
        extra = xchg > staged ? xchg : staged;
    } else if (o_dtype == KDA_BF16) {
        extra = rows * V * 4;           // bf16 results staged in fp32
    }
    return extra ? ((base + 255) & ~(size_t)255) + extra : base;
}

}  // extern "C"

namespace {

kda_status_t chunk_fwd_stages(int stages, const char *name,
                              const void *q, const void *k, const void *v,
                              const float *g, const float *beta_raw,
                              const float *A_log, const float *dt_bias,
                              float scale, float lower_bound,
                              const int64_t *cu_seqlens, int32_t num_seqs,
                              int64_t total_tokens, int32_t H, int32_t K, int32_t V,
                              int32_t chunk_size, kda_dtype_t in_dtype,
                              const float *initial_state, float *final_state,
                              void *o, kda_dtype_t o_dtype,
                              void *workspace, size_t workspace_bytes,
                              void *stream, int32_t H_qk, bool fixed_scratch = false,
                              const void *z = nullptr, const float *norm_weight = nullptr,
                              float norm_eps = 0.f) {
    if (num_seqs < 1) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 1");
    if (total_tokens < 0) return fail(KDA_ERR_INVALID_ARG, "total_tokens must be >= 0");
    // the head size the kernels run at: K = V natively, or both padded to it
    const int native = native_head_size(K, V, chunk_size, in_dtype);
    const int D = native ? native : padded_head_size(K, V, chunk_size, in_dtype);
    if (D == 0 && K >= 1 && V >= 1 && K <= 256 && V <= 256)
        return fail(KDA_ERR_UNSUPPORTED, "K or V above 128 needs chunk_size 64 and bf16 inputs (got K=" +
                                             std::to_string(K) + ", V=" + std::to_string(V) +
                                             "; kda_recurrent_fwd takes any K, V up to 256)");
    kda_status_t st = check_common(H, D == 256 ? std::min(K, 128) : K, D == 256 ? std::min(V, 128) : V,
                                   scale, lower_bound, in_dtype, o_dtype, true);
    if (st != KDA_OK) return st;
    st = check_groups(H, H_qk);
    if (st != KDA_OK) return st;
    if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64)
        return fail(KDA_ERR_UNSUPPORTED, "chunk_size must be 16, 32 or 64");
    if (!cu_seqlens || !A_log || !dt_bias)
        return fail(KDA_ERR_INVALID_ARG, "cu_seqlens, A_log and dt_bias must not be NULL");
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta_raw || !o))
        return fail(KDA_ERR_INVALID_ARG, "q, k, v, g, beta_raw and o must not be NULL");
    if ((int64_t)num_seqs * H > (int64_t)1 << 28)
        return fail(KDA_ERR_INVALID_ARG, "num_seqs * H too large");
    if (kda::num_slots(total_tokens, num_seqs, chunk_size) > ((int64_t)1 << 31) - 1)
        return fail(KDA_ERR_INVALID_ARG, "too many chunks for one launch");
    const size_t need = z ? kda_chunk_fwd_gated_workspace_size(total_tokens, num_seqs, H, K, V,
                                                               chunk_size, in_dtype, o_dtype)
                          : kda_chunk_fwd_workspace_size(total_tokens, num_seqs, H, K, V,
                                                         chunk_size, in_dtype);
    if (fixed_scratch) {
        if (need > kda::kNoAllocScratchBytes)
            return fail(KDA_ERR_WORKSPACE,
                        std::string(name) + ": these sizes need " + std::to_string(need) +
                            " bytes of scratch, above its fixed " +
                            std::to_string(kda::kNoAllocScratchBytes) +
                            " bytes; call kda_chunk_fwd with a caller workspace");
    } else {
        if (!workspace || workspace_bytes < need)
            return fail(KDA_ERR_WORKSPACE, "workspace needs " + std::to_string(need) +
                                               " bytes, got " + std::to_string(workspace_bytes));
        if (((uintptr_t)workspace & 255) != 0)
            return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }
    st = check_aligned16({{q, "q"}, {k, "k"}, {v, "v"}, {g, "g"}, {dt_bias, "dt_bias"},
                          {initial_state, "initial_state"}, {final_state, "final_state"},
                          {o, "o"}});
    if (st != KDA_OK) return st;
    if (((uintptr_t)beta_raw & 3) != 0 || ((uintptr_t)A_log & 3) != 0)
        return fail(KDA_ERR_INVALID_ARG, "beta_raw and A_log must be 4-byte aligned");
    if (z) {
        if (stages != 3) return fail(KDA_ERR_INVALID_ARG, "the output epilogue runs with both stages");
        if (!norm_weight) return fail(KDA_ERR_INVALID_ARG, "norm_weight must not be NULL");
        if (!(norm_eps > 0.0f) || !std::isfinite(norm_eps))
            return fail(KDA_ERR_INVALID_ARG, "norm_eps must be finite and > 0");
        st = check_aligned16({{z, "z"}, {norm_weight, "norm_weight"}});
        if (st != KDA_OK) return st;
        const uintptr_t esz = in_dtype == KDA_BF16 ? 2 : 4, osz = o_dtype == KDA_BF16 ? 2 : 4;
        if (overlaps(byte_range(z, (uintptr_t)total_tokens * H * V * esz),
                     byte_range(o, (uintptr_t)total_tokens * H * V * osz)))
            return fail(KDA_ERR_INVALID_ARG, "z and o must not overlap");
    }
    if (fixed_scratch) {
        // every argument check has passed: the current device's copy of the
        // library's fixed scratch array replaces the caller workspace
        const hipError_t e = kda::noalloc_scratch(&workspace);
        if (e != hipSuccess) return hip_fail(e, name);
        workspace_bytes = kda::kNoAllocScratchBytes;
    }

    kda::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta_raw = beta_raw; a.A_log = A_log; a.dt_bias = dt_bias;
    a.scale = scale; a.lower_bound = lower_bound;
    a.cu_seqlens = cu_seqlens; a.N = num_seqs; a.T = total_tokens; a.H = H; a.Hk = H_qk;
    a.chunk = chunk_size;
    a.h0 = initial_state; a.ht = final_state; a.o = o;
    a.in_bf16 = in_dtype == KDA_BF16; a.out_bf16 = o_dtype == KDA_BF16;
    a.ws = (unsigned char *)workspace;
    a.stream = (hipStream_t)stream;
    a.stages = stages;
    // The output epilogue, when asked for. The natively sized K = V = 128
    // kernels with 64-row chunks of bf16 inputs apply it in the inter-chunk
    // kernel when all of that kernel's workgroups fit the GPU at once (the two
    // workgroups of a chain exchange row sums through the workspace, after the
    // part kda_chunk_fwd uses). Otherwise it is a pass over the V-wide output
    // rows right after the inter-chunk kernel on the same stream (the outputs
    // are still in the memory-side cache then), reading them unrounded: fp32
    // results in place, bf16 results staged in the workspace after the part
    // kda_chunk_fwd uses, so that y is rounded once.
    unsigned char *const extra =
        z ? (unsigned char *)workspace +
                ((kda_chunk_fwd_workspace_size(total_tokens, num_seqs, H, K, V, chunk_size,
                                               in_dtype) + 255) & ~(size_t)255)
          : nullptr;
    bool fuse = false;
    if (z && native == 128 && total_tokens > 0) {
        kda::PrefillArgs t = a;
        t.D = native;
        const hipError_t e = kda::prefill_gate_fusable(t, fuse);
        if (e != hipSuccess) return hip_fail(e, name);
    }
    const bool stage_o = z && !fuse && o_dtype == KDA_BF16;
    unsigned char *const o32 = stage_o ? extra : nullptr;
    // The natively sized K = V = 128 kernels with 64-row chunks and bf16 inputs
    // stage the outputs in half the bytes: fp16 with a power-of-two scale per
    // 16-feature block of each row (T x H x 8 fp32 scales after the rows).
    const bool stage_h = stage_o && native == 128 && chunk_size == 64 && in_dtype == KDA_BF16;
    float *const o_sc =
        stage_h ? (float *)(o32 + (size_t)total_tokens * H * V * sizeof(uint16_t)) : nullptr;
    auto epilogue = [&]() -> hipError_t {
        if (!z || fuse || total_tokens == 0) return hipSuccess;
        kda::NormGateArgs ng;
        ng.o = stage_o ? (const void *)o32 : o; ng.z = z; ng.w = norm_weight; ng.eps = norm_eps;
        ng.o_scale = o_sc;
        ng.rows = total_tokens * H; ng.D = V;
        ng.bf16 = !stage_o && o_dtype == KDA_BF16; ng.z_bf16 = in_dtype == KDA_BF16;
        ng.y_bf16 = o_dtype == KDA_BF16; ng.y = o;
        ng.stream = (hipStream_t)stream;
        return kda::launch_norm_gate(ng);
    };
    if (stage_o) a.out_bf16 = false;
    if (native) {
        a.D = native;
        if (fuse) {
            a.z = z; a.norm_w = norm_weight; a.norm_eps = norm_eps;
            a.xchg = (uint64_t *)extra;
        }
        if (stage_o) a.o = o32;
        a.o_scale = o_sc;
        hipError_t e = kda::launch_prefill(a);
        if (e == hipSuccess) e = epilogue();
        if (e != hipSuccess) return hip_fail(e, name);
        return ok();
    }

    // other sizes: the kernels for D on zero-padded copies in the workspace
    a.D = D;
    const int esz = in_dtype == KDA_BF16 ? 2 : 4, osz = o_dtype == KDA_BF16 ? 2 : 4;
    const PadLayout P = pad_layout(total_tokens, num_seqs, H,
                                   in_dtype, kda_chunk_fwd_workspace_size(total_tokens, num_seqs, H,
                                                                          D, D, chunk_size,
                                                                          in_dtype),
                                   (size_t)D);
    unsigned char *ws = (unsigned char *)workspace;
    hipStream_t s = a.stream;
    const int64_t TH = total_tokens * H, THk = total_tokens * H_qk, NH = (int64_t)num_seqs * H;
    hipError_t e = hipSuccess;
    auto pad = [&](const void *src, int sc, int64_t rs, void *dst, int dc, int64_t rd, int64_t rows,
                   int bytes) {
        if (e == hipSuccess) e = kda::launch_pad_rows(src, sc, rs, dst, dc, rd, rows, bytes, s);
    };
    if (stages & 1) {
        pad(q, K, 1, ws + P.q, D, 1, THk, esz);
        pad(k, K, 1, ws + P.k, D, 1, THk, esz);
        pad(v, V, 1, ws + P.v, D, 1, TH, esz);
        pad(g, K, 1, ws + P.g, D, 1, TH, 4);
        pad(dt_bias, K, 1, ws + P.dtb, D, 1, H, 4);
    }
    if ((stages & 2) && initial_state)                 // value rows widened to D as well
        pad(initial_state, K, V, ws + P.state, D, D, NH * D, 4);
    if (e != hipSuccess) return hip_fail(e, name);
    a.q = ws + P.q; a.k = ws + P.k; a.v = ws + P.v; a.g = (const float *)(ws + P.g);
    a.dt_bias = (const float *)(ws + P.dtb);
    a.h0 = initial_state ? (const float *)(ws + P.state) : nullptr;
    a.ht = final_state ? (float *)(ws + P.state) : nullptr;     // read before written, per block
    a.o = ws + P.o;
    e = kda::launch_prefill(a);
    if (e != hipSuccess) return hip_fail(e, name);
    if (stages & 2) {
        if (stage_o) pad(ws + P.o, D, 1, o32, V, 1, TH, 4);
        else pad(ws + P.o, D, 1, o, V, 1, TH, osz);
        if (final_state) pad(ws + P.state, D, D, final_state, K, V, NH * V, 4);
        if (e == hipSuccess) e = epilogue();
        if (e != hipSuccess) return hip_fail(e, name);
    }
    return ok();
}

}  // namespace

extern "C" {

#define KDA_CHUNK_ARGS                                                                     \
    q, k, v, g, beta_raw, A_log, dt_bias, scale, lower_bound, cu_seqlens, num_seqs,       \
        total_tokens, H, K, V, chunk_size, in_dtype, initial_state, final_state, o,        \
        o_dtype, workspace, workspace_bytes, stream
#define KDA_CHUNK_PARAMS                                                                   \
    const void *q, const void *k, const void *v, const float *g, const float *beta_raw,    \
        const float *A_log, const float *dt_bias, float scale, float lower_bound,          \
        const int64_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens, int32_t H,      \
        int32_t K, int32_t V, int32_t chunk_size, kda_dtype_t in_dtype,                    \
        const float *initial_state, float *final_state, void *o, kda_dtype_t o_dtype,      \
        void *workspace, size_t workspace_bytes, void *stream

kda_status_t kda_chunk_fwd(KDA_CHUNK_PARAMS) {
    return chunk_fwd_stages(3, "kda_chunk_fwd", KDA_CHUNK_ARGS, H);
}

kda_status_t kda_chunk_fwd_intra(KDA_CHUNK_PARAMS) {
    return chunk_fwd_stages(1, "kda_chunk_fwd_intra", KDA_CHUNK_ARGS, H);
}

kda_status_t kda_chunk_fwd_inter(KDA_CHUNK_PARAMS) {
    return chunk_fwd_stages(2, "kda_chunk_fwd_inter", KDA_CHUNK_ARGS, H);
}

kda_status_t kda_chunk_fwd_grouped(KDA_CHUNK_PARAMS, int32_t H_qk) {
    return chunk_fwd_stages(3, "kda_chunk_fwd_grouped", KDA_CHUNK_ARGS, H_qk);
}

kda_status_t kda_chunk_fwd_gated(KDA_CHUNK_PARAMS, const void *z, const float *norm_weight,
                                 float norm_eps) {
    if (!z && total_tokens > 0) return fail(KDA_ERR_INVALID_ARG, "z must not be NULL");
    return chunk_fwd_stages(3, "kda_chunk_fwd_gated", KDA_CHUNK_ARGS, H, false, z, norm_weight,
                            norm_eps);
}

kda_status_t kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                   const float *g, const float *beta_raw,
                                   const float *A_log, const float *dt_bias,
                                   float scale, float lower_bound,
                                   const int64_t *cu_seqlens, int32_t num_seqs,
                                   int64_t total_tokens, int32_t H, int32_t K, int32_t V,
                                   int32_t chunk_size, kda_dtype_t in_dtype,
                                   const float *initial_state, float *final_state,
                                   void *o, kda_dtype_t o_dtype, void *stream) {
    return chunk_fwd_stages(3, "kda_chunk_fwd_noalloc", q, k, v, g, beta_raw, A_log, dt_bias,
                            scale, lower_bound, cu_seqlens, num_seqs, total_tokens, H, K, V,
                            chunk_size, in_dtype, initial_state, final_state, o, o_dtype,
                            nullptr, 0, stream, H, /*fixed_scratch=*/true);
}

kda_status_t kda_decode_step_grouped(const void *q, const void *k, const void *v,
                                     const float *g, const float *beta_raw,
                                     const float *A_log, const float *dt_bias,
                                     float scale, float lower_bound,
                                     float *state, int32_t num_slots, const int32_t *slot_idx,
                                     void *o, kda_dtype_t o_dtype,
                                     int32_t B, int32_t H, int32_t H_qk, int32_t K, int32_t V,
                                     kda_dtype_t in_dtype,
                                     const void *z, const float *norm_weight, float norm_eps,
                                     void *stream) {
    if (slot_idx) {
        if (num_slots < 1) return fail(KDA_ERR_INVALID_ARG, "num_slots must be >= 1");
        if (((uintptr_t)slot_idx & 3) != 0) return fail(KDA_ERR_INVALID_ARG, "slot_idx must be 4-byte aligned");
        if ((int64_t)num_slots * H > ((int64_t)1 << 31) - 1)
            return fail(KDA_ERR_INVALID_ARG, "num_slots * H too large");
    }
    return decode_step_impl(q, k, v, g, beta_raw, A_log, dt_bias, scale, lower_bound, state, o,
                            o_dtype, B, H, K, V, in_dtype, stream, z, norm_weight, norm_eps,
                            slot_idx, slot_idx ? num_slots : 0, "kda_decode_step_grouped launch",
                            H_qk);
}


kda_status_t kda_decode_step(const void *q, const void *k, const void *v,
                             const float *g, const float *beta_raw,
                             const float *A_log, const float *dt_bias,
                             float scale, float lower_bound,
                             float *state, void *o, kda_dtype_t o_dtype,
                             int32_t B, int32_t H, int32_t K, int32_t V,
                             kda_dtype_t in_dtype, void *stream) {
    return decode_step_impl(q, k, v, g, beta_raw, A_log, dt_bias, scale, lower_bound, state, o,
                            o_dtype, B, H, K, V, in_dtype, stream, nullptr, nullptr, 0.f,
                            nullptr, 0, "kda_decode_step launch", H);
}

kda_status_t kda_decode_step_gated(const void *q, const void *k, const void *v,
                                   const float *g, const float *beta_raw,
                                   const float *A_log, const float *dt_bias,
                                   float scale, float lower_bound,
                                   float *state, void *o, kda_dtype_t o_dtype,
                                   int32_t B, int32_t H, int32_t K, int32_t V,
                                   kda_dtype_t in_dtype,
                                   const void *z, const float *norm_weight, float norm_eps,
                                   void *stream) {
    if (!z) return fail(KDA_ERR_INVALID_ARG, "z is NULL");
    return decode_step_impl(q, k, v, g, beta_raw, A_log, dt_bias, scale, lower_bound, state, o,
                            o_dtype, B, H, K, V, in_dtype, stream, z, norm_weight, norm_eps,
                            nullptr, 0, "kda_decode_step_gated launch", H);
}

kda_status_t kda_decode_step_slots(const void *q, const void *k, const void *v,
                                   const float *g, const float *beta_raw,
                                   const float *A_log, const float *dt_bias,
                                   float scale, float lower_bound,
                                   float *state_pool, int32_t num_slots, const int32_t *slot_idx,
                                   void *o, kda_dtype_t o_dtype,
                                   int32_t B, int32_t H, int32_t K, int32_t V,
                                   kda_dtype_t in_dtype,
                                   const void *z, const float *norm_weight, float norm_eps,
                                   void *stream) {
    if (num_slots < 1) return fail(KDA_ERR_INVALID_ARG, "num_slots must be >= 1");
    if (!slot_idx) return fail(KDA_ERR_INVALID_ARG, "slot_idx is NULL");
    if (((uintptr_t)slot_idx & 3) != 0) return fail(KDA_ERR_INVALID_ARG, "slot_idx must be 4-byte aligned");
    if ((int64_t)num_slots * H > ((int64_t)1 << 31) - 1)
        return fail(KDA_ERR_INVALID_ARG, "num_slots * H too large");
    return decode_step_impl(q, k, v, g, beta_raw, A_log, dt_bias, scale, lower_bound, state_pool,
                            o, o_dtype, B, H, K, V, in_dtype, stream, z, norm_weight, norm_eps,
                            slot_idx, num_slots, "kda_decode_step_slots launch", H);
}

kda_status_t kda_output_norm_gate(const void *o, const void *z, const float *weight, float eps,
                                  int64_t rows, int32_t D, kda_dtype_t io_dtype, void *y,
                                  void *stream) {
    if (rows < 0) return fail(KDA_ERR_INVALID_ARG, "rows must be >= 0");
    if (D < 1 || D > 256) return fail(KDA_ERR_UNSUPPORTED, "D must lie in [1, 256] (got " + std::to_string(D) + ")");
    if (!valid_dtype(io_dtype)) return fail(KDA_ERR_UNSUPPORTED, "unknown dtype");
    if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(KDA_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (rows == 0) return ok();                 // nothing to read or write (pointers may be NULL)
    if (!o || !z || !weight || !y) return fail(KDA_ERR_INVALID_ARG, "a required pointer is NULL");
    if ((rows + 3) / 4 > (int64_t)0x7fffffff) return fail(KDA_ERR_INVALID_ARG, "rows too large");
    kda_status_t st = check_aligned16({{o, "o"}, {z, "z"}, {weight, "weight"}, {y, "y"}});
    if (st != KDA_OK) return st;
    kda::NormGateArgs a;
    a.o = o; a.z = z; a.w = weight; a.eps = eps; a.rows = rows; a.D = D; a.bf16 = io_dtype == KDA_BF16;
    a.z_bf16 = a.bf16; a.y_bf16 = a.bf16;
    a.y = y; a.stream = (hipStream_t)stream;
    hipError_t e = kda::launch_norm_gate(a);
    if (e != hipSuccess) return hip_fail(e, "kda_output_norm_gate launch");
    return ok();
}

kda_status_t kda_short_conv(const void *x, int64_t x_stride, const float *weight, int32_t W,
                            const int64_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                            int64_t channels, kda_dtype_t dtype, const void *state_in,
                            void *state_out, void *y, void *stream) {
    kda_status_t st = check_short_conv(x, x_stride, weight, W, cu_seqlens, num_seqs, total_tokens,
                                       channels, dtype, y);
    if (st != KDA_OK) return st;
    if (W == 1) { state_in = nullptr; state_out = nullptr; }   // no history to carry
    st = check_aligned16({{x, "x"}, {y, "y"}, {state_in, "state_in"}, {state_out, "state_out"}});
    if (st != KDA_OK) return st;
    // y is written while x and the carried-in state are read by other threads,
    // so no output may overlap an input; the final state may only be the
    // carried-in state itself (updated in place)
    const bool bf16 = dtype == KDA_BF16;
    const uintptr_t es = bf16 ? 2 : 4;
    const ByteRange rx = total_tokens > 0 ? byte_range(x, ((uintptr_t)(total_tokens - 1) * x_stride + channels) * es) : ByteRange{};
    const ByteRange ry = byte_range(y, (uintptr_t)total_tokens * channels * es);
    const uintptr_t sbytes = (uintptr_t)num_seqs * (W - 1) * channels * es;
    const ByteRange rsi = byte_range(state_in, sbytes), rso = byte_range(state_out, sbytes);
    if (overlaps(ry, rx) || overlaps(ry, rsi) || overlaps(ry, rso))
        return fail(KDA_ERR_INVALID_ARG, "y must not overlap x or a conv state");
    if (overlaps(rso, rx) || (overlaps(rso, rsi) && state_out != state_in))
        return fail(KDA_ERR_INVALID_ARG, "state_out must not overlap x, and may overlap state_in only by being it");

    kda::ShortConvArgs a;
    a.x = x; a.x_stride = x_stride; a.w = weight; a.W = W; a.cu = cu_seqlens; a.N = num_seqs;
    a.T = total_tokens; a.channels = channels; a.st_in = state_in; a.st_out = state_out; a.y = y;
    a.bf16 = bf16; a.stream = (hipStream_t)stream;
    hipError_t e = kda::launch_short_conv(a);
    if (e != hipSuccess) return hip_fail(e, "kda_short_conv launch");
    return ok();
}

kda_status_t kda_short_conv_slots(const void *x, int64_t x_stride, const float *weight, int32_t W,
                                  const int64_t *cu_seqlens, int32_t num_seqs,
                                  int64_t total_tokens, int64_t channels, kda_dtype_t dtype,
                                  void *state_pool, int32_t num_slots, const int32_t *slot_idx,
                                  void *y, void *stream) {
    kda_status_t st = check_short_conv(x, x_stride, weight, W, cu_seqlens, num_seqs, total_tokens,
                                       channels, dtype, y);
    if (st != KDA_OK) return st;
    if (num_slots < 1) return fail(KDA_ERR_INVALID_ARG, "num_slots must be >= 1");
    if (!slot_idx) return fail(KDA_ERR_INVALID_ARG, "slot_idx is NULL");
    if (((uintptr_t)slot_idx & 3) != 0) return fail(KDA_ERR_INVALID_ARG, "slot_idx must be 4-byte aligned");
    if (W > 1 && !state_pool) return fail(KDA_ERR_INVALID_ARG, "state_pool is NULL");
    if (W == 1) state_pool = nullptr;
    st = check_aligned16({{x, "x"}, {y, "y"}, {state_pool, "state_pool"}});
    if (st != KDA_OK) return st;
    const bool bf16 = dtype == KDA_BF16;
    const uintptr_t es = bf16 ? 2 : 4;
    const ByteRange rx = total_tokens > 0 ? byte_range(x, ((uintptr_t)(total_tokens - 1) * x_stride + channels) * es) : ByteRange{};
    const ByteRange ry = byte_range(y, (uintptr_t)total_tokens * channels * es);
    const ByteRange rp = byte_range(state_pool, (uintptr_t)num_slots * (W - 1) * channels * es);
    if (overlaps(ry, rx) || overlaps(ry, rp) || overlaps(rp, rx))
        return fail(KDA_ERR_INVALID_ARG, "y, x and state_pool must not overlap");

    kda::ShortConvArgs a;
    a.x = x; a.x_stride = x_stride; a.w = weight; a.W = W; a.cu = cu_seqlens; a.N = num_seqs;
    a.T = total_tokens; a.channels = channels; a.st_in = state_pool; a.st_out = state_pool; a.y = y;
    a.slots = slot_idx; a.num_slots = num_slots; a.bf16 = bf16; a.stream = (hipStream_t)stream;
    hipError_t e = kda::launch_short_conv(a);
    if (e != hipSuccess) return hip_fail(e, "kda_short_conv_slots launch");
    return ok();
}

size_t kda_backward_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                   int32_t K, int32_t V) {
    if (total_tokens < 0 || num_seqs < 1 || H < 1 || H > 65535) {
        fail(KDA_ERR_INVALID_ARG, "need total_tokens >= 0, num_seqs >= 1, 1 <= H <= 65535");
        return 0;
    }
    if (K < 1 || K > 128 || V < 1 || V > 128) {
        fail(KDA_ERR_UNSUPPORTED, "K and V must lie in [1, 128]");
        return 0;
    }
    g_last_error.clear();
    const size_t base = kda::backward_layout(total_tokens, num_seqs, H).total;
    if (K == 128 && V == 128) return base;
    return bwd_pad_layout(total_tokens, num_seqs, H, base).end;
}

kda_status_t kda_backward_grouped(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta_raw, const float *A_log, const float *dt_bias,
                                  float scale, float lower_bound, const int64_t *cu_seqlens,
                                  int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t H_qk,
                                  int32_t K, int32_t V, kda_dtype_t in_dtype,
                                  const float *initial_state, const void *d_o, kda_dtype_t do_dtype,
                                  const float *d_final_state, float *dq, float *dk, float *dv,
                                  float *dg, float *dbeta, float *dA_log, float *ddt_bias,
                                  float *d_initial_state, void *workspace, size_t workspace_bytes,
                                  void *stream) {
    if (num_seqs < 1) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 1");
    if (total_tokens < 0) return fail(KDA_ERR_INVALID_ARG, "total_tokens must be >= 0");
    if (H > 65535) return fail(KDA_ERR_INVALID_ARG, "H must lie in [1, 65535]");
    kda_status_t st = check_common(H, K, V, scale, lower_bound, in_dtype, do_dtype, true);
    if (st != KDA_OK) return st;
    st = check_groups(H, H_qk);
    if (st != KDA_OK) return st;
    if (!cu_seqlens || !A_log || !dt_bias || !dA_log || !ddt_bias)
        return fail(KDA_ERR_INVALID_ARG, "cu_seqlens, A_log, dt_bias, dA_log and ddt_bias must not be NULL");
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta_raw || !d_o || !dq || !dk || !dv ||
                             !dg || !dbeta))
        return fail(KDA_ERR_INVALID_ARG, "a token tensor or its gradient is NULL");
    if ((int64_t)num_seqs * H > (int64_t)1 << 28)
        return fail(KDA_ERR_INVALID_ARG, "num_seqs * H too large");
    if ((total_tokens + 15) / 16 > (int64_t)0x7fffffff)
        return fail(KDA_ERR_INVALID_ARG, "total_tokens too large");
    const size_t need = kda_backward_workspace_size(total_tokens, num_seqs, H, K, V);
    if (!workspace || workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes, got " +
                                           std::to_string(workspace_bytes));
    if (((uintptr_t)workspace & 255) != 0)
        return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    st = check_aligned16({{q, "q"}, {k, "k"}, {v, "v"}, {g, "g"}, {dt_bias, "dt_bias"},
                          {initial_state, "initial_state"}, {d_o, "d_o"},
                          {d_final_state, "d_final_state"}, {dq, "dq"}, {dk, "dk"}, {dv, "dv"},
                          {dg, "dg"}, {ddt_bias, "ddt_bias"}, {d_initial_state, "d_initial_state"}});
    if (st != KDA_OK) return st;
    if (((uintptr_t)beta_raw & 3) != 0 || ((uintptr_t)A_log & 3) != 0 ||
        ((uintptr_t)dbeta & 3) != 0 || ((uintptr_t)dA_log & 3) != 0)
        return fail(KDA_ERR_INVALID_ARG, "beta_raw, A_log, dbeta and dA_log must be 4-byte aligned");

    const kda::BackwardLayout lay = kda::backward_layout(total_tokens, num_seqs, H);
    kda::BackwardArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta_raw = beta_raw; a.A_log = A_log; a.dt_bias = dt_bias;
    a.scale = scale; a.lower_bound = lower_bound; a.cu = cu_seqlens; a.N = num_seqs; a.H = H;
    a.Hk = H_qk; a.T = total_tokens; a.in_bf16 = in_dtype == KDA_BF16; a.do_bf16 = do_dtype == KDA_BF16;
    a.h0 = initial_state; a.dout = d_o; a.dht = d_final_state;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dA_log = dA_log;
    a.ddt_bias = ddt_bias; a.dh0 = d_initial_state;
    unsigned char *ws = (unsigned char *)workspace;
    a.ckpt = (float *)ws;
    a.pp = (float *)(ws + lay.ckpt_bytes);
    a.ops = (float *)(ws + lay.ckpt_bytes + lay.pp_bytes);
    a.rr = (float *)(ws + lay.ckpt_bytes + lay.pp_bytes + lay.ops_bytes);
    a.stream = (hipStream_t)stream;
    if (K == 128 && V == 128) {
        hipError_t e = kda::launch_backward(a);
        if (e != hipSuccess) return hip_fail(e, "kda_backward launch");
        return ok();
    }

    // below 128: the same kernels on zero-padded copies (as kda_chunk_fwd). The
    // padded channels and rows stay zero in the forward, so the gradients of
    // the real inputs are those of the K x V problem; the padded ones are dropped.
    const int64_t D = kda::kHeadDimHost;
    const int esz = in_dtype == KDA_BF16 ? 2 : 4, dsz = do_dtype == KDA_BF16 ? 2 : 4;
    const BwdPadLayout P = bwd_pad_layout(total_tokens, num_seqs, H, lay.total);
    const int64_t TH = total_tokens * H, THk = total_tokens * H_qk, NH = (int64_t)num_seqs * H;
    hipStream_t s = a.stream;
    hipError_t e = hipSuccess;
    auto pad = [&](const void *src, int sc, int64_t rs, void *dst, int dc, int64_t rd, int64_t rows,
                   int bytes) {
        if (e == hipSuccess) e = kda::launch_pad_rows(src, sc, rs, dst, dc, rd, rows, bytes, s);
    };
    pad(q, K, 1, ws + P.q, D, 1, THk, esz);
    pad(k, K, 1, ws + P.k, D, 1, THk, esz);
    pad(v, V, 1, ws + P.v, D, 1, TH, esz);
    pad(g, K, 1, ws + P.g, D, 1, TH, 4);
    pad(dt_bias, K, 1, ws + P.dtb, D, 1, H, 4);
    if (initial_state) pad(initial_state, K, V, ws + P.h0, D, D, NH * D, 4);
    pad(d_o, V, 1, ws + P.dout, D, 1, TH, dsz);
    if (d_final_state) pad(d_final_state, K, V, ws + P.dht, D, D, NH * D, 4);
    if (e != hipSuccess) return hip_fail(e, "kda_backward padding");
    a.q = ws + P.q; a.k = ws + P.k; a.v = ws + P.v; a.g = (const float *)(ws + P.g);
    a.dt_bias = (const float *)(ws + P.dtb);
    a.h0 = initial_state ? (const float *)(ws + P.h0) : nullptr;
    a.dout = ws + P.dout;
    a.dht = d_final_state ? (const float *)(ws + P.dht) : nullptr;
    a.dq = (float *)(ws + P.dq); a.dk = (float *)(ws + P.dk); a.dv = (float *)(ws + P.dv);
    a.dg = (float *)(ws + P.dg); a.ddt_bias = (float *)(ws + P.ddt);
    a.dh0 = d_initial_state ? (float *)(ws + P.dh0) : nullptr;
    e = kda::launch_backward(a);
    if (e != hipSuccess) return hip_fail(e, "kda_backward launch");
    pad(ws + P.dq, D, 1, dq, K, 1, THk, 4);
    pad(ws + P.dk, D, 1, dk, K, 1, THk, 4);
    pad(ws + P.dv, D, 1, dv, V, 1, TH, 4);
    pad(ws + P.dg, D, 1, dg, K, 1, TH, 4);
    pad(ws + P.ddt, D, 1, ddt_bias, K, 1, H, 4);
    if (d_initial_state) pad(ws + P.dh0, D, D, d_initial_state, K, V, NH * V, 4);
    if (e != hipSuccess) return hip_fail(e, "kda_backward padding");
    return ok();
}

kda_status_t kda_backward(const void *q, const void *k, const void *v, const float *g,
                          const float *beta_raw, const float *A_log, const float *dt_bias,
                          float scale, float lower_bound, const int64_t *cu_seqlens,
                          int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t K, int32_t V,
                          kda_dtype_t in_dtype, const float *initial_state, const void *d_o,
                          kda_dtype_t do_dtype, const float *d_final_state, float *dq, float *dk,
                          float *dv, float *dg, float *dbeta, float *dA_log, float *ddt_bias,
                          float *d_initial_state, void *workspace, size_t workspace_bytes,
                          void *stream) {
    return kda_backward_grouped(q, k, v, g, beta_raw, A_log, dt_bias, scale, lower_bound,
                                cu_seqlens, num_seqs, total_tokens, H, H, K, V, in_dtype,
                                initial_state, d_o, do_dtype, d_final_state, dq, dk, dv, dg, dbeta,
                                dA_log, ddt_bias, d_initial_state, workspace, workspace_bytes,
                                stream);
}

kda_status_t kda_recurrent_fwd(const void *q, const void *k, const void *v,
                               const float *g, const float *beta_raw,
                               const float *A_log, const float *dt_bias,
                               float scale, float lower_bound,
                               const int64_t *cu_seqlens, int32_t num_seqs,
                               int64_t total_tokens, int32_t H, int32_t H_qk,
                               int32_t K, int32_t V, kda_dtype_t in_dtype,
                               const float *initial_state, float *final_state,
                               void *o, kda_dtype_t o_dtype, void *stream) {
    if (H < 1 || H > 65536) return fail(KDA_ERR_INVALID_ARG, "H must lie in [1, 65536]");
    kda_status_t st = check_groups(H, H_qk);
    if (st != KDA_OK) return st;
    if (K < 1 || K > 256 || V < 1 || V > 256)
        return fail(KDA_ERR_UNSUPPORTED, "K and V must lie in [1, 256] (got K=" + std::to_string(K) +
                                             ", V=" + std::to_string(V) + ")");
    if (!(scale > 0.0f) || !std::isfinite(scale))
        return fail(KDA_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (!(lower_bound >= -5.0f && lower_bound < 0.0f))
        return fail(KDA_ERR_INVALID_ARG, "lower_bound must lie in [-5, 0)");
    if (!valid_dtype(in_dtype)) return fail(KDA_ERR_UNSUPPORTED, "unknown input dtype");
    if (!valid_dtype(o_dtype)) return fail(KDA_ERR_UNSUPPORTED, "unknown output dtype");
    if (num_seqs < 1) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 1");
    if (total_tokens < 0) return fail(KDA_ERR_INVALID_ARG, "total_tokens must be >= 0");
    if (!A_log || !dt_bias || !cu_seqlens)
        return fail(KDA_ERR_INVALID_ARG, "A_log, dt_bias and cu_seqlens must not be NULL");
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta_raw || !o))
        return fail(KDA_ERR_INVALID_ARG, "a token pointer is NULL");
    const uintptr_t te = in_dtype == KDA_BF16 ? 1 : 3, oe = o_dtype == KDA_BF16 ? 1 : 3;
    if (((uintptr_t)q & te) || ((uintptr_t)k & te) || ((uintptr_t)v & te) || ((uintptr_t)o & oe) ||
        ((uintptr_t)g & 3) || ((uintptr_t)beta_raw & 3) || ((uintptr_t)A_log & 3) ||
        ((uintptr_t)dt_bias & 3) || ((uintptr_t)initial_state & 3) || ((uintptr_t)final_state & 3) ||
        ((uintptr_t)cu_seqlens & 7))
        return fail(KDA_ERR_INVALID_ARG, "a pointer is not aligned to its element size");
    const size_t sbytes = (size_t)num_seqs * H * V * K * 4;
    const ByteRange rsi = byte_range(initial_state, sbytes), rso = byte_range(final_state, sbytes);
    if (overlaps(rsi, rso) && initial_state != final_state)
        return fail(KDA_ERR_INVALID_ARG, "final_state may overlap initial_state only by being it");
    if (kda::general_blocks(num_seqs, H, V) > (int64_t)0x7fffffff)
        return fail(KDA_ERR_INVALID_ARG, "num_seqs * H * V too large for one launch");

    kda::GeneralArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta_raw = beta_raw; a.A_log = A_log; a.dt_bias = dt_bias;
    a.scale = scale; a.lower_bound = lower_bound; a.cu_seqlens = cu_seqlens;
    a.N = num_seqs; a.H = H; a.Hk = H_qk; a.K = K; a.V = V;
    a.h0 = initial_state; a.ht = final_state; a.o = o;
    a.in_bf16 = in_dtype == KDA_BF16; a.out_bf16 = o_dtype == KDA_BF16;
    a.stream = (hipStream_t)stream;
    const hipError_t e = kda::launch_recurrent_fwd(a);
    if (e != hipSuccess) return hip_fail(e, "kda_recurrent_fwd launch");
    return ok();
}

kda_status_t kda_stream_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (bytes == 0) return ok();
    if (!src || !dst) return fail(KDA_ERR_INVALID_ARG, "src and dst must not be NULL");
    if (bytes % 16 != 0) return fail(KDA_ERR_INVALID_ARG, "bytes must be a multiple of 16");
    kda_status_t st = check_aligned16({{src, "src"}, {dst, "dst"}});
    if (st != KDA_OK) return st;
    if (overlaps(byte_range(src, bytes), byte_range(dst, bytes)))
        return fail(KDA_ERR_INVALID_ARG, "src and dst overlap");
    const hipError_t e = kda::launch_stream_copy(src, dst, bytes, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "kda_stream_copy");
    return ok();
}

kda_status_t kda_check_cu_seqlens(const int64_t *cu_seqlens, int32_t num_seqs,
                                  int64_t total_tokens, void *stream) {
    if (!cu_seqlens || num_seqs < 1 || total_tokens < 0)
        return fail(KDA_ERR_INVALID_ARG, "need cu_seqlens != NULL, num_seqs >= 1, total_tokens >= 0");
    std::vector<int64_t> h((size_t)num_seqs + 1);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(h.data(), cu_seqlens, h.size() * sizeof(int64_t),
                                  hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "kda_check_cu_seqlens copy");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "kda_check_cu_seqlens sync");
    if (h[0] != 0) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens[0] != 0");
    for (int32_t i = 0; i < num_seqs; ++i)
        if (h[i + 1] < h[i])
            return fail(KDA_ERR_INVALID_ARG, "cu_seqlens decreases at index " + std::to_string(i));
    if (h[num_seqs] != total_tokens)
        return fail(KDA_ERR_INVALID_ARG, "cu_seqlens[num_seqs] != total_tokens");
    return ok();
}

}  // extern "C"
