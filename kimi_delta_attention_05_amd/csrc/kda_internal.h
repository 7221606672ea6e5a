// Internal interfaces of libkda: launch arguments and the workspace record layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kHeadDimHost = 128;    // the head size the chunkwise and decode kernels are built for

struct DecodeArgs {
    const void *q, *k, *v;
    const float *g, *beta_raw, *A_log, *dt_bias;
    float scale, lower_bound;
    float *state;
    void *o;
    int B, H;
    int Hk = 0;                         // q/k heads (grouped value heads), as PrefillArgs
    bool in_bf16, out_bf16;
    hipStream_t stream;
    // output epilogue fused into the store (z == nullptr: none): RMS norm with
    // channel weight norm_w, then the sigmoid gate of logits z (input dtype)
    const void *z = nullptr;
    const float *norm_w = nullptr;
    float norm_eps = 0.f;
    // state pool addressing (slots == nullptr: state is [B, H, V, K]): request b
    // uses pool entry slots[b] (device int32), padding if outside [0, num_slots)
    const int32_t *slots = nullptr;
    int num_slots = 0;
};

// Output epilogue over rows of 128 features: y = o / sqrt(mean(o^2) + eps) * w * sigmoid(z).
struct NormGateArgs {
    const void *o, *z;
    const float *w;
    float eps;
    int64_t rows;
    int D = 128;                        // features per row (128, or any width up to 256)
    bool bf16;                          // dtype of o
    // when set (D = 128): o is fp16, each row's 16-value block to be multiplied by
    // o_scale [rows, 8]
    const float *o_scale = nullptr;
    bool z_bf16 = false;                // dtype of z
    bool y_bf16 = false;                // dtype of y
    void *y;
    hipStream_t stream;
};

struct PrefillArgs {
    const void *q, *k, *v;
    const float *g, *beta_raw, *A_log, *dt_bias;
    float scale, lower_bound;
    const int64_t *cu_seqlens;
    int N;
    int64_t T;
    int H;               // value heads (v, g, beta, states, o)
    int Hk = 0;          // q/k heads (H a multiple of it; value head h reads q/k head h / (H / Hk))
    int chunk;
    const float *h0;
    float *ht;
    void *o;
    bool in_bf16, out_bf16;
    unsigned char *ws;
    hipStream_t stream;
    int stages;          // bit 0: intra-chunk kernel, bit 1: inter-chunk kernel
    int D = 128;         // head size K = V: 128, or 64 or 256 (64-row chunks of bf16 inputs only)
    // when set (D = 128, 64-row chunks, bf16 inputs): o is fp16, each row's 16-value
    // block divided by the power of two in o_scale [T, H, D / 16]
    float *o_scale = nullptr;
    // when z is set (D = 128, 64-row chunks, bf16 inputs, both stages; see
    // prefill_gate_fusable): o receives y = o / sqrt(mean(o^2) + norm_eps) *
    // norm_w * sigmoid(z) per row, z [T, H, 128] bf16, norm_w [128]; xchg: the
    // halves' row-sum exchange, num_slots * H * 128 words of workspace
    const void *z = nullptr;
    const float *norm_w = nullptr;
    float norm_eps = 0.f;
    uint64_t *xchg = nullptr;
};

// Geometry of one chunk of C rows (C = 16, 32 or 64).
template <int C>
struct ChunkGeom {
    static constexpr int NB = C / 16;            // 16-row blocks
    static constexpr int CP = C < 32 ? 32 : C;   // t extent rounded up to whole 32-wide k-steps
    static constexpr int CS = CP / 32;           // 32-wide k-steps over t
};

// One workspace record per (chunk slot, head). Everything the inter-chunk
// kernel needs, stored in MFMA operand order so that each lane reads 16 (or 32)
// contiguous bytes per fragment:
//   -W   [NB tb][4 s][64 lane][8]   rows t, k over key channels   (Tst), negated
//                                   so that U = Ub + (-W) S^T is one accumulation
//   qg   [NB tb][4 s][64 lane][8]   rows t, k over key channels   (Tst)
//   kgT  [8 kb][CS s][64 lane][8]   rows key channel, k over t    (Tst)
// A fragment's lane l holds row l % 16; its 8 k-values are, for k over key
// channels, the channels 32 s + 8 (l / 16) + e, and for k over t the rows
// 32 s + kperm(l / 16, e) (kda_common.h). Row r of kgT tile kb is the key
// channel tile_chan(kb, r), so that the state tiles the inter-chunk kernel
// accumulates from it stack into the channel order of W and qg.
//   M    [NB tb][CS s][64 lane][8]  rows t, k over t'             (Tst); fragments
//                                   with 2 s > tb lie above the diagonal, are
//                                   never read and are left unwritten
//   GamC [128]                      fp32 total decay of the chunk
//   UbSc [4]                        fp32; [0] = power-of-two scale of Ub, 0 if
//                                   every v of the chunk is zero
//   Ub   [8 vb][NB tb][64 lane][4]  accumulator tiles of T V / UbSc[0] (Tub)
// Rows past the end of a partial chunk are zero in -W, kgT and Ub (so they add
// nothing to U or the state); in qg and M they are unspecified (they reach
// only output rows that are never stored).
// Tst and Tub are fp16 when the inputs are bf16 (W, qg, kg, M are bounded by 1
// in magnitude; Ub is stored scaled so that it is bounded by 2^15) and fp32
// when the inputs are fp32.
// The head size D (K = V = D) is 128 or, for the natively sized 64-row bf16
// kernels, 64: the arrays above then hold D / 32 k-steps over key channels
// (KS), D / 16 key-channel tiles of kg^T (KT) and D / 16 value blocks of Ub
// (VT) instead of 4, 8 and 8.
template <int C, bool PRECISE, int D = 128>
struct Record {
    using G = ChunkGeom<C>;
    static constexpr int KS = D / 32, KT = D / 16, VT = D / 16;
    static constexpr size_t ELT = PRECISE ? 4 : 2;
    static constexpr size_t FRAG = 64 * 8 * ELT;
    static constexpr size_t W_OFF = 0;
    static constexpr size_t QG_OFF = W_OFF + (size_t)G::NB * KS * FRAG;
    static constexpr size_t KG_OFF = QG_OFF + (size_t)G::NB * KS * FRAG;
    static constexpr size_t M_OFF = KG_OFF + (size_t)KT * G::CS * FRAG;
    static constexpr size_t GC_OFF = M_OFF + (size_t)G::NB * G::CS * FRAG;
    static constexpr size_t UBS_OFF = GC_OFF + D * 4;
    static constexpr size_t SHARED_BYTES = UBS_OFF + 16;
    static constexpr size_t UB_OFF = SHARED_BYTES;
    static constexpr size_t UB_ELT = PRECISE ? 4 : 2;
    static constexpr size_t UB_VB_BYTES = (size_t)G::NB * 64 * 4 * UB_ELT;
    static constexpr size_t BYTES = UB_OFF + VT * UB_VB_BYTES;
};

size_t record_bytes(int chunk, bool precise, int D = 128);

// Number of chunk slots: chunk j of sequence n lives in slot floor(cu[n]/C) + n + j,
// which is unique and below floor(T/C) + N for any valid offsets.
__host__ __device__ inline int64_t num_slots(int64_t T, int N, int chunk) { return T / chunk + N; }

// Front end: causal depthwise short conv + SiLU over `channels` channels.
struct ShortConvArgs {
    const void *x = nullptr;            // [T] rows of `channels`, row stride x_stride
    int64_t x_stride = 0;               // elements
    const float *w = nullptr;           // [channels, W]
    int W = 0;                          // 1 .. 4
    const int64_t *cu = nullptr;        // [N + 1] device offsets
    int N = 0;
    int64_t T = 0;
    int64_t channels = 0;               // multiple of 8
    const void *st_in = nullptr;        // [N, W - 1, channels] or NULL (zero history)
    void *st_out = nullptr;             // [N, W - 1, channels] or NULL; may equal st_in
    void *y = nullptr;                  // [T, channels]
    // state pool addressing (slots == nullptr: states indexed by sequence): sequence
    // n uses pool entry slots[n] (device int32), padding if outside [0, num_slots);
    // st_in == st_out == the pool
    const int32_t *slots = nullptr;
    int num_slots = 0;
    bool bf16 = false;
    hipStream_t stream = nullptr;
};

// Training backward of the recurrence (all gradients fp32).
struct BackwardArgs {
    const void *q, *k, *v;              // [T, H, 128] input dtype
    const float *g, *beta_raw, *A_log, *dt_bias;
    float scale, lower_bound;
    const int64_t *cu;                  // [N + 1]
    int N, H;
    int Hk = 0;                         // q/k heads (grouped value heads), as PrefillArgs
    int64_t T;
    bool in_bf16, do_bf16;
    const float *h0;                    // [N, H, 128, 128] or NULL (zero)
    const void *dout;                   // [T, H, 128] output adjoint
    const float *dht;                   // [N, H, 128, 128] final-state adjoint or NULL (zero)
    float *dq, *dk, *dv, *dg, *dbeta, *dA_log, *ddt_bias;
    float *dh0;                         // or NULL
    float *ckpt, *pp, *ops, *rr;        // workspace pieces (backward_layout)
    hipStream_t stream;
};

struct BackwardLayout {
    size_t ckpt_bytes, pp_bytes, ops_bytes, rr_bytes, total;
};
BackwardLayout backward_layout(int64_t T, int N, int H);
hipError_t launch_backward(const BackwardArgs &a);

// Workgroups of the two front-end launches (for the host's size checks).
int64_t short_conv_blocks(int64_t T, int64_t channels, bool bf16);
int64_t short_conv_state_blocks(int64_t N, int64_t channels);

// Recurrent forward for any head sizes K, V in [1, 256] (token by token, fp32).
struct GeneralArgs {
    const void *q, *k, *v;
    const float *g, *beta_raw, *A_log, *dt_bias;
    float scale, lower_bound;
    const int64_t *cu_seqlens;          // nullptr: one token per sequence (sequence n = token n)
    int N, H, Hk, K, V;
    const float *h0;
    float *ht;
    void *o;
    bool in_bf16, out_bf16;
    hipStream_t stream;
    // state pool (decode only, cu_seqlens == nullptr): sequence n's state is pool
    // entry slots[n]; an entry outside [0, num_slots) marks a padding request
    const int32_t *slots = nullptr;
    int num_slots = 0;
};
int64_t general_blocks(int64_t N, int64_t H, int V);
// dst row d = src row (d / rd) * rs + d % rd if d % rd < rs (first min(src_cols,
// dst_cols) elements, zeros after), else zeros; elements of 2 or 4 bytes
hipError_t launch_pad_rows(const void *src, int src_cols, int64_t rs, void *dst, int dst_cols,
                           int64_t rd, int64_t dst_rows, int elem_bytes, hipStream_t stream);
hipError_t launch_recurrent_fwd(const GeneralArgs &a);

// Fixed scratch of kda_chunk_fwd_noalloc: a file-scope device array of this many
// bytes per GPU; noalloc_scratch returns the current device's copy (looked up
// once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;
hipError_t noalloc_scratch(void **ptr);

hipError_t launch_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

hipError_t launch_decode(const DecodeArgs &a);
hipError_t launch_norm_gate(const NormGateArgs &a);
hipError_t prefill_gate_fusable(const PrefillArgs &a, bool &fusable);
hipError_t launch_prefill(const PrefillArgs &a);
hipError_t launch_short_conv(const ShortConvArgs &a);

}  // namespace kda
