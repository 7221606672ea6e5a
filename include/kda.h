/*
 * libkda — Kimi Delta Attention (KDA) forward on AMD MI355X (gfx950).
 *
 * C ABI. Plain pointers and sizes only; every tensor pointer is device memory
 * owned by the caller. The library never allocates or frees device memory and
 * never synchronises inside kda_chunk_fwd or kda_decode_step: all work is
 * enqueued on the caller's HIP stream and the call returns at once.
 *
 * What is computed (FlashInfer "kda_backward" page, "Supported contract"; the
 * kda-neuron-kernels commit log for the per-key-channel decay): for every
 * sequence and head, a value-first fp32 state S[V][K] evolves token by token as
 *
 *   qh = q / sqrt(|q|^2 + 1e-6) * scale        kh = k / sqrt(|k|^2 + 1e-6)
 *   alpha_c = exp(lower_bound * sigmoid(exp(A_log[h]) * (g_c + dt_bias[h,c])))
 *   b = sigmoid(beta_raw)
 *   S <- S diag(alpha)                          decay each key channel (column)
 *   S <- S + b (v - S kh) kh^T                  delta-rule write
 *   o  = S qh                                   read after the write
 *
 * Layouts (row-major, packed along the token axis, B = 1 for prefill):
 *   q, k, g : [T, H, K]      v, o : [T, H, V]      beta_raw : [T, H]
 *   A_log   : [H] fp32       dt_bias : [H, K] fp32
 *   states  : [N, H, V, K] fp32 (value-first)
 * K and V are 128 (the contract's head dimension) except where an entry point
 * says otherwise (kda_chunk_fwd and kda_backward: 1..128; kda_recurrent_fwd and
 * the plain decode step: 1..256); 1 <= H <= 65536. g, beta_raw,
 * A_log, dt_bias and the states are always fp32; q, k and v share the input
 * dtype; o has its own dtype.
 *
 * Alignment: q, k, v, g, dt_bias, o and the states must be 16-byte aligned,
 * beta_raw and A_log 4-byte aligned (any allocation from hipMalloc is);
 * a misaligned pointer is rejected with KDA_ERR_INVALID_ARG.
 *
 * Errors: every entry point returns a status. Argument checks run on the host
 * before any HIP call; a failed check enqueues nothing. kda_last_error() gives
 * a human-readable detail for the last failure on the calling thread.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,   /* NULL pointer, negative size, bad scale or bound */
    KDA_ERR_UNSUPPORTED = 2,   /* head size outside the entry point's range, chunk not in {16,32,64}, bad dtype */
    KDA_ERR_WORKSPACE = 3,     /* workspace NULL or smaller than required */
    KDA_ERR_HIP = 4            /* a HIP launch or runtime call failed */
} kda_status_t;

typedef enum {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype_t;

/* Library ABI version (major * 100 + minor). */
int kda_version(void);

/* Static text for a status code. */
const char *kda_status_string(kda_status_t status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char *kda_last_error(void);

/*
 * Bytes of device workspace kda_chunk_fwd needs for these sizes, or 0 if the
 * arguments are invalid (then kda_last_error() says why). The workspace holds
 * the per-chunk intermediates of the chunkwise form (one record per chunk slot
 * and head; there are floor(T / chunk_size) + num_seqs slots) and is fully
 * rewritten by every call, so it may be reused across calls on one stream.
 */
size_t kda_chunk_fwd_workspace_size(int64_t total_tokens, int32_t num_seqs,
                                    int32_t H, int32_t K, int32_t V,
                                    int32_t chunk_size, kda_dtype_t in_dtype);

/*
 * Chunkwise prefill over packed variable-length sequences.
 * (kimi_k3 FusedKDAChunkwise page, "Exact upstream call contract": the
 * chunk_kda call with in-kernel L2 normalisation, gate and sigmoid beta, safe
 * gate, lower bound, chunk size and value-first state; FlashInfer kda_backward
 * page for dtypes, layouts and packed int64 offsets.)
 *
 * q, k, v      : [T, H, 128] in in_dtype (KDA_BF16 or KDA_F32)
 * g            : [T, H, 128] fp32 raw gate;  beta_raw : [T, H] fp32
 * A_log        : [H] fp32;  dt_bias : [H, 128] fp32
 * scale        : output scale (> 0), normally 1/sqrt(128)
 * lower_bound  : gate floor in [-5, 0); -5 in the contract
 * cu_seqlens   : DEVICE pointer to num_seqs + 1 int64 offsets with cu[0] = 0,
 *                non-decreasing, cu[num_seqs] = total_tokens. The values are a
 *                precondition and are not checked here (see
 *                kda_check_cu_seqlens); the kernels read them directly.
 * initial_state: [num_seqs, H, 128, 128] fp32, or NULL for zero states
 * final_state  : [num_seqs, H, 128, 128] fp32, or NULL to skip. May alias
 *                initial_state (each workgroup reads its slice before writing).
 * o            : [T, H, 128] in o_dtype (KDA_BF16 or KDA_F32), rounded to
 *                nearest even when bf16
 * chunk_size   : 16, 32 or 64 (the model validator admits 32 and 64; 16 is
 *                also accepted). The result does not depend on it beyond
 *                rounding.
 * workspace    : device memory of at least kda_chunk_fwd_workspace_size(...)
 *                bytes, 256-byte aligned; contents on entry are ignored.
 * stream       : hipStream_t to enqueue on (NULL = default stream).
 * A zero-length sequence writes no output rows and copies its initial state
 * (or zeros) to its final state. total_tokens = 0 is allowed.
 *
 * Other head sizes (FlashKDA issue page, "Proposed scope": arbitrary
 * key/value dimensions): K and V may each be 1..128, and 1..256 with
 * chunk_size 64 and bf16 inputs (otherwise KDA_ERR_UNSUPPORTED;
 * kda_recurrent_fwd takes any K, V up to 256), with q, k, g [T, H, K],
 * v, o [T, H, V], dt_bias [H, K] and states [num_seqs, H, V, K]. K = V = 64
 * and K = V = 256 with chunk_size 64 and bf16 inputs run on kernels sized
 * for them. Other sizes run the 128-wide kernels (K, V <= 128) or the
 * 256-wide ones (K or V above 128) on copies padded with zeros to that many
 * key channels and value rows, which kda_chunk_fwd_workspace_size includes in
 * the workspace: padded channels and rows stay exactly zero through the
 * recurrence, so the result is that of the K x V problem.
 */
kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v,
                           const float *g, const float *beta_raw,
                           const float *A_log, const float *dt_bias,
                           float scale, float lower_bound,
                           const int64_t *cu_seqlens, int32_t num_seqs,
                           int64_t total_tokens, int32_t H, int32_t K, int32_t V,
                           int32_t chunk_size, kda_dtype_t in_dtype,
                           const float *initial_state, float *final_state,
                           void *o, kda_dtype_t o_dtype,
                           void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * The two stages of kda_chunk_fwd, callable separately with the same
 * arguments and the same workspace (kda_chunk_fwd = intra, then inter, on one
 * stream). kda_chunk_fwd_intra reads q, k, v, g, beta_raw, A_log, dt_bias and
 * cu_seqlens and fills the workspace with the per-chunk intermediates; it is
 * parallel over all chunks and heads. kda_chunk_fwd_inter reads the workspace,
 * cu_seqlens and initial_state and writes o and final_state; it walks the
 * chunks of each sequence in order (the "all chunks in one launch, state kept
 * on chip" design of the kda-neuron-kernels fused chunked forward). Between
 * the two calls the workspace must not be modified. Splitting lets a caller
 * overlap the intra stage with other work or time the stages separately.
 */
kda_status_t kda_chunk_fwd_intra(const void *q, const void *k, const void *v,
                                 const float *g, const float *beta_raw,
                                 const float *A_log, const float *dt_bias,
                                 float scale, float lower_bound,
                                 const int64_t *cu_seqlens, int32_t num_seqs,
                                 int64_t total_tokens, int32_t H, int32_t K, int32_t V,
                                 int32_t chunk_size, kda_dtype_t in_dtype,
                                 const float *initial_state, float *final_state,
                                 void *o, kda_dtype_t o_dtype,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);
kda_status_t kda_chunk_fwd_inter(const void *q, const void *k, const void *v,
                                 const float *g, const float *beta_raw,
                                 const float *A_log, const float *dt_bias,
                                 float scale, float lower_bound,
                                 const int64_t *cu_seqlens, int32_t num_seqs,
                                 int64_t total_tokens, int32_t H, int32_t K, int32_t V,
                                 int32_t chunk_size, kda_dtype_t in_dtype,
                                 const float *initial_state, float *final_state,
                                 void *o, kda_dtype_t o_dtype,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * One T=1 decode step for B independent requests, all heads in one launch.
 * (kda-neuron-kernels commit log: batched multi-(request, head) decode and the
 * one-pass "key-fold" recurrent step; same transforms as above.)
 *
 * q, k, v  : [B, H, 128] in in_dtype;  g : [B, H, 128] fp32;  beta_raw : [B, H]
 * state    : [B, H, 128, 128] fp32, read and updated in place
 * o        : [B, H, 128] in o_dtype
 * The state is read once and written once per step.
 * Other head sizes (1 <= K, V <= 256, FlashKDA issue page, "Proposed scope"):
 * q, k, g [B, H, K], v, o [B, H, V], state [B, H, V, K], run by the
 * token-by-token kernel of kda_recurrent_fwd with one token per request; every
 * decode form accepts them (the output epilogue, whose row then spans several
 * of the step's workgroups, runs as a second pass over o: norm_weight [V], z
 * [B, H, V]; the rows (B * H) must fit 4 per workgroup in one launch).
 */
kda_status_t kda_decode_step(const void *q, const void *k, const void *v,
                             const float *g, const float *beta_raw,
                             const float *A_log, const float *dt_bias,
                             float scale, float lower_bound,
                             float *state, void *o, kda_dtype_t o_dtype,
                             int32_t B, int32_t H, int32_t K, int32_t V,
                             kda_dtype_t in_dtype, void *stream);

/*
 * kda_decode_step with the output epilogue of kda_output_norm_gate fused into
 * its output store (each (request, head) row of 128 outputs is normalised,
 * weighted and gated before it is written; the same arithmetic as running
 * kda_output_norm_gate on o afterwards, without the extra pass over o).
 *
 * z           : [B, H, 128] gate logits in in_dtype, 16-byte aligned, not NULL
 * norm_weight : [128] fp32, 16-byte aligned;  norm_eps : finite and > 0
 * Every other argument as for kda_decode_step.
 */
kda_status_t kda_decode_step_gated(const void *q, const void *k, const void *v,
                                   const float *g, const float *beta_raw,
                                   const float *A_log, const float *dt_bias,
                                   float scale, float lower_bound,
                                   float *state, void *o, kda_dtype_t o_dtype,
                                   int32_t B, int32_t H, int32_t K, int32_t V,
                                   kda_dtype_t in_dtype,
                                   const void *z, const float *norm_weight, float norm_eps,
                                   void *stream);
/*
 * Serving form of the decode step: the states live in a pool of num_slots
 * entries and request b uses entry slot_idx[b], so that a batch can be formed
 * from any subset of live sequences without moving states (continuous
 * batching); everything else as for kda_decode_step, with the output epilogue
 * of kda_decode_step_gated when z is not NULL. Makes no allocation, copy or
 * synchronisation, so it can be captured in a HIP graph and replayed with new
 * contents in the same buffers.
 *
 * state_pool : [num_slots, H, 128, 128] fp32, 16-byte aligned; the entries
 *              named by slot_idx are read and updated in place
 * slot_idx   : DEVICE pointer to B int32 slot indices, 4-byte aligned. A
 *              request whose index lies outside [0, num_slots) is padding: its
 *              output row is written as zeros and no state is touched. Two
 *              requests naming the same slot in one call race (undefined
 *              result).
 * z, norm_weight, norm_eps : as for kda_decode_step_gated, or z = NULL for the
 *              plain step (norm_weight and norm_eps are then ignored)
 */
kda_status_t kda_decode_step_slots(const void *q, const void *k, const void *v,
                                   const float *g, const float *beta_raw,
                                   const float *A_log, const float *dt_bias,
                                   float scale, float lower_bound,
                                   float *state_pool, int32_t num_slots, const int32_t *slot_idx,
                                   void *o, kda_dtype_t o_dtype,
                                   int32_t B, int32_t H, int32_t K, int32_t V,
                                   kda_dtype_t in_dtype,
                                   const void *z, const float *norm_weight, float norm_eps,
                                   void *stream);
/*
 * Output epilogue of the attention block (kimi_k3 FusedKDAChunkwise page,
 * "Output handling": the per-head output norm, then the sigmoid output gate
 * whose logits are a projection of the hidden states; that projection and the
 * output projection after it need model weights and are not part of libkda).
 * For each row r of D = 128 features:
 *
 *   y[r, c] = o[r, c] / sqrt(mean_c' o[r, c']^2 + eps) * weight[c] * sigmoid(z[r, c])
 *
 * computed in fp32 and rounded to nearest even when bf16. For a prefill output
 * rows = total_tokens * H ([T, H, 128] viewed as [T * H, 128]).
 *
 * o, z, y : [rows, 128] in io_dtype (KDA_BF16 or KDA_F32), 16-byte aligned;
 *           y may alias o
 * weight  : [128] fp32 (one weight vector shared by all heads), 16-byte aligned
 * eps     : finite and > 0 (the page gives no value)
 * rows    : >= 0 (0 enqueues nothing and accepts NULL pointers);  D : 128, or any
 *           width 1..256 for the outputs of other head sizes (o, z, y [rows, D],
 *           weight [D]; a slower one-wave-per-row kernel)
 */
kda_status_t kda_output_norm_gate(const void *o, const void *z, const float *weight, float eps,
                                  int64_t rows, int32_t D, kda_dtype_t io_dtype, void *y,
                                  void *stream);
/*
 * Front end of the attention block (kimi_k3 FusedKDAChunkwise page, "CUDA-only
 * forward and causal preprocessing": after the q, k, v projections each channel
 * is left-padded by W - 1 along time, filtered by its own depthwise kernel and
 * passed through SiLU). Call it once each for q, k and v, with their own
 * weights. For each channel c and token t of packed sequence n:
 *
 *   y[t, c] = silu( sum_{i=0}^{W-1} weight[c, i] * x[t - (W - 1) + i, c] ),  silu(u) = u sigmoid(u)
 *
 * where the W - 1 positions before the sequence's first token are rows of its
 * carried-in conv state (oldest first), or zeros when state_in is NULL; tap
 * W - 1 multiplies the current token. Computed in fp32, rounded to nearest
 * even when bf16.
 *
 * x         : total_tokens rows of `channels` elements in dtype, row stride
 *             x_stride elements (>= channels, a multiple of 8; a slice of a
 *             fused projection output can be passed as it is), 16-byte aligned
 * weight    : [channels, W] fp32 (the layout of a grouped conv1d weight
 *             [channels, 1, W]), 4-byte aligned
 * W         : kernel size, 1 .. 4 (the page gives none)
 * cu_seqlens: [num_seqs + 1] int64 DEVICE offsets, trusted as for kda_chunk_fwd
 * channels  : H * 128 for one of q, k, v; a positive multiple of 8
 * state_in  : [num_seqs, W - 1, channels] in dtype, or NULL (zero history)
 * state_out : [num_seqs, W - 1, channels] in dtype, or NULL: each sequence's
 *             last W - 1 inputs, reaching back into state_in for sequences
 *             shorter than W - 1 (an empty sequence passes its state on). May
 *             be state_in itself (updated in place). Both are ignored when W == 1.
 * y         : [total_tokens, channels] in dtype, contiguous, 16-byte aligned
 *
 * y may not overlap x or a state, and state_out may not overlap x or partly
 * overlap state_in: rejected with KDA_ERR_INVALID_ARG. total_tokens == 0 only
 * passes states on (x and y may then be NULL).
 */
kda_status_t kda_short_conv(const void *x, int64_t x_stride, const float *weight, int32_t W,
                            const int64_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                            int64_t channels, kda_dtype_t dtype, const void *state_in,
                            void *state_out, void *y, void *stream);
/*
 * Serving form of kda_short_conv: the conv states live in a pool of num_slots
 * entries and sequence n uses entry slot_idx[n], read as its carried-in state
 * and replaced by its final state (one decode token per request is a sequence
 * of length 1; a prefill chunk continues a request's earlier chunks). A
 * sequence whose index lies outside [0, num_slots) is padding: its outputs are
 * written as zeros and no state is read or written. Two sequences naming the
 * same entry in one call race (undefined result).
 *
 * state_pool : [num_slots, W - 1, channels] in dtype, 16-byte aligned, updated
 *              in place (ignored when W == 1); must not overlap x or y
 * slot_idx   : DEVICE pointer to num_seqs int32 entries, 4-byte aligned
 * Everything else as for kda_short_conv. Makes no allocation, copy or
 * synchronisation.
 */
kda_status_t kda_short_conv_slots(const void *x, int64_t x_stride, const float *weight, int32_t W,
                                  const int64_t *cu_seqlens, int32_t num_seqs,
                                  int64_t total_tokens, int64_t channels, kda_dtype_t dtype,
                                  void *state_pool, int32_t num_slots, const int32_t *slot_idx,
                                  void *y, void *stream);
/*
 * Training backward of the recurrence (FlashInfer kda_backward page,
 * "Supported contract": gradients for q, k, v, the raw gate, raw beta, A_log,
 * dt_bias and the initial state, given the output adjoint; its persistent
 * forward-checkpoint + reverse design). With S the state, the forward per
 * token being S' = S diag(alpha), u = b (v - S' kh), S <- S' + u kh^T,
 * o = S qh, the gradients are those of the loss sum(o * d_o) +
 * sum(final_state * d_final_state) with respect to every input, computed in
 * fp32 (fp32 MFMA products and sums) in the chunked form of the recurrence
 * over 16-token chunks: a forward pass stores the state at every chunk start
 * in the workspace, a reverse pass carries the state adjoint across chunks, and
 * the per-chunk gradients follow from the chunk's operands and the reverse
 * pass's per-chunk sums. Workspace at T = 8192, N = 1, H = 96: 5.2 GB (per
 * 16-token chunk and head: the 64 KiB checkpoint, a 30.5 KiB operand record and
 * 8 KiB of the forward's intermediate values).
 *
 * Inputs as for kda_chunk_fwd (q, k, v in in_dtype; g, beta_raw, A_log,
 * dt_bias, initial_state fp32; initial_state may be NULL = zero), plus
 *   d_o           : [T, H, 128] output adjoint in do_dtype
 *   d_final_state : [N, H, 128, 128] fp32 adjoint of the final state, or NULL (zero)
 * Outputs, all fp32 and fully overwritten:
 *   dq, dk, dg    : [T, H, 128]      dv : [T, H, 128]      dbeta : [T, H] (w.r.t. beta_raw)
 *   dA_log        : [H]              ddt_bias : [H, 128]   (summed over all sequences)
 *   d_initial_state : [N, H, 128, 128], or NULL to skip
 * workspace: kda_backward_workspace_size() bytes, 256-byte aligned, caller
 * owned; nothing in it needs initialising. H <= 65535. Sums run in a fixed
 * order (no atomics): results repeat bit for bit.
 * Head sizes below 128 (1 <= K, V <= 128; shapes as for kda_chunk_fwd, d_o
 * [T, H, V], d_final_state and d_initial_state [N, H, V, K]): the same kernels
 * on zero-padded copies in the workspace, as kda_chunk_fwd does; the gradients
 * of the padded channels and rows are dropped.
 */
size_t kda_backward_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                   int32_t K, int32_t V);
kda_status_t kda_backward(const void *q, const void *k, const void *v, const float *g,
                          const float *beta_raw, const float *A_log, const float *dt_bias,
                          float scale, float lower_bound, const int64_t *cu_seqlens,
                          int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t K, int32_t V,
                          kda_dtype_t in_dtype, const float *initial_state, const void *d_o,
                          kda_dtype_t do_dtype, const float *d_final_state, float *dq, float *dk,
                          float *dv, float *dg, float *dbeta, float *dA_log, float *ddt_bias,
                          float *d_initial_state, void *workspace, size_t workspace_bytes,
                          void *stream);
/*
 * Any head sizes (FlashKDA issue page, "Proposed scope": arbitrary key/value
 * dimensions). The recurrence above for 1 <= K <= 256 and 1 <= V <= 256, computed
 * token by token in fp32 by one kernel (the chunkwise path and the decode
 * kernels require K = V = 128). Packed variable-length sequences with offsets
 * cu_seqlens as for kda_chunk_fwd; grouped value heads as below (H_qk == H:
 * ungrouped). A batched decode step is this call with cu_seqlens = [0, 1, ..., B]
 * and the request states as initial_state / final_state.
 *   q, k : [T, H_qk, K]   v, o : [T, H, V]   g : [T, H, K]   beta_raw : [T, H]
 *   A_log : [H]   dt_bias : [H, K]   states : [N, H, V, K] fp32 (value-first)
 * initial_state NULL = zero; final_state NULL = not written; final_state may be
 * initial_state itself (updated in place; any other overlap is rejected).
 * Pointers need only their element alignment (cu_seqlens 8 bytes). A sequence
 * of length 0 writes no output and copies its initial state (or zeros) to
 * final_state. Enqueued on `stream`; no workspace.
 */
kda_status_t kda_recurrent_fwd(const void *q, const void *k, const void *v,
                               const float *g, const float *beta_raw,
                               const float *A_log, const float *dt_bias,
                               float scale, float lower_bound,
                               const int64_t *cu_seqlens, int32_t num_seqs,
                               int64_t total_tokens, int32_t H, int32_t H_qk,
                               int32_t K, int32_t V, kda_dtype_t in_dtype,
                               const float *initial_state, float *final_state,
                               void *o, kda_dtype_t o_dtype, void *stream);
/*
 * Grouped value heads (FlashKDA issue page, "Proposed scope": grouped value
 * heads). H value heads share H_qk query/key heads, H a multiple of H_qk: value
 * head h reads q and k of head h / (H / H_qk). v, g, beta_raw, the states and
 * the outputs keep H heads; q and k are [T, H_qk, K] (decode: [B, H_qk, K]).
 * The same computation as the ungrouped call with q and k repeated H / H_qk
 * times along the head axis; H_qk == H is the ungrouped call. Everything else
 * as for kda_chunk_fwd, kda_decode_step_slots / _gated / plain, and
 * kda_backward; H_qk that does not divide H is rejected with
 * KDA_ERR_INVALID_ARG. In kda_backward_grouped dq and dk are [T, H_qk, K],
 * summed over the value heads of each group.
 *
 * kda_decode_step_grouped covers the three decode forms: slot_idx NULL for a
 * state [B, H, V, K] (num_slots ignored), else a pool of num_slots entries
 * addressed as in kda_decode_step_slots; z NULL for no output epilogue.
 */
kda_status_t kda_chunk_fwd_grouped(const void *q, const void *k, const void *v,
                                   const float *g, const float *beta_raw,
                                   const float *A_log, const float *dt_bias,
                                   float scale, float lower_bound,
                                   const int64_t *cu_seqlens, int32_t num_seqs,
                                   int64_t total_tokens, int32_t H, int32_t K, int32_t V,
                                   int32_t chunk_size, kda_dtype_t in_dtype,
                                   const float *initial_state, float *final_state,
                                   void *o, kda_dtype_t o_dtype,
                                   void *workspace, size_t workspace_bytes, void *stream,
                                   int32_t H_qk);
kda_status_t kda_decode_step_grouped(const void *q, const void *k, const void *v,
                                     const float *g, const float *beta_raw,
                                     const float *A_log, const float *dt_bias,
                                     float scale, float lower_bound,
                                     float *state, int32_t num_slots, const int32_t *slot_idx,
                                     void *o, kda_dtype_t o_dtype,
                                     int32_t B, int32_t H, int32_t H_qk, int32_t K, int32_t V,
                                     kda_dtype_t in_dtype,
                                     const void *z, const float *norm_weight, float norm_eps,
                                     void *stream);
kda_status_t kda_backward_grouped(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta_raw, const float *A_log, const float *dt_bias,
                                  float scale, float lower_bound, const int64_t *cu_seqlens,
                                  int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t H_qk,
                                  int32_t K, int32_t V, kda_dtype_t in_dtype,
                                  const float *initial_state, const void *d_o, kda_dtype_t do_dtype,
                                  const float *d_final_state, float *dq, float *dk, float *dv,
                                  float *dg, float *dbeta, float *dA_log, float *ddt_bias,
                                  float *d_initial_state, void *workspace, size_t workspace_bytes,
                                  void *stream);
/*
 * kda_chunk_fwd with the output epilogue of kda_output_norm_gate applied in
 * the o store (kimi_k3 FusedKDAChunkwise page, "Output handling": per-head norm
 * of each output row, then the sigmoid output gate): o receives
 *   y = o_kda / sqrt(mean(o_kda^2) + norm_eps) * norm_weight * sigmoid(z)
 * computed in fp32 from the fp32 outputs and rounded once to o_dtype. z: [T, H, V] gate
 * logits in in_dtype (must not overlap o; may be NULL only when
 * total_tokens = 0); norm_weight: [V] fp32; norm_eps finite and > 0. Other
 * arguments, layouts and errors as kda_chunk_fwd, with the workspace sized by
 * kda_chunk_fwd_gated_workspace_size. The rows of one output come from two
 * workgroups of the inter-chunk kernel (one per half of the state). With
 * K = V = 128, chunk_size 64 and bf16 inputs, when the batch's N * H chains
 * fit the GPU at once (two workgroups each, one per CU), that kernel applies
 * the epilogue itself: the two workgroups of a chain exchange their halves'
 * row sums of squares through the workspace. Otherwise the epilogue is a pass
 * over the outputs right after the inter-chunk kernel: fp32 results in
 * place, bf16 results staged in the workspace, in fp32, or at K = V = 128,
 * chunk 64, bf16 inputs in fp16 with a power-of-two scale per 16 features
 * (each value then within 2^-11 of its 16 features' largest magnitude).
 */
/* Workspace bytes kda_chunk_fwd_gated needs: kda_chunk_fwd_workspace_size,
 * rounded up to 256, plus, at K = V = 128 with chunk_size 64 and bf16 inputs,
 * the larger of the row-sum exchange (8 * 128 * H * (T / 64 + N) bytes) and,
 * for bf16 o, the staged outputs (T * H * (2 V + V / 4) bytes); in other
 * configurations, for bf16 o, T * H * V * 4 bytes of fp32 staging (nothing for
 * fp32 o). 0 for invalid arguments. */
size_t kda_chunk_fwd_gated_workspace_size(int64_t total_tokens, int32_t num_seqs,
                                          int32_t H, int32_t K, int32_t V,
                                          int32_t chunk_size, kda_dtype_t in_dtype,
                                          kda_dtype_t o_dtype);
kda_status_t kda_chunk_fwd_gated(const void *q, const void *k, const void *v,
                                 const float *g, const float *beta_raw,
                                 const float *A_log, const float *dt_bias,
                                 float scale, float lower_bound,
                                 const int64_t *cu_seqlens, int32_t num_seqs,
                                 int64_t total_tokens, int32_t H, int32_t K, int32_t V,
                                 int32_t chunk_size, kda_dtype_t in_dtype,
                                 const float *initial_state, float *final_state,
                                 void *o, kda_dtype_t o_dtype,
                                 void *workspace, size_t workspace_bytes, void *stream,
                                 const void *z, const float *norm_weight, float norm_eps);
/*
 * kda_chunk_fwd without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Arguments and results as kda_chunk_fwd; the
 * workspace is a fixed device array inside the library of 128 MiB per GPU
 * (134217728 bytes), allocated when the library's code is loaded on a device
 * and held until the process ends. Sizes whose
 * kda_chunk_fwd_workspace_size exceeds it (e.g. T = 8192 at H = 12 fits,
 * T = 8192 at H = 96 does not) are rejected with KDA_ERR_WORKSPACE before any
 * HIP call. The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); its first call on a device looks up that device's copy of
 * the array. Every call on one GPU shares that GPU's array and it keeps the
 * last call's contents (the kernels rewrite everything they read, so nothing
 * needs clearing): calls that overlap on one GPU (other streams, other
 * threads) race and give undefined results; serialise them.
 */
kda_status_t kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                   const float *g, const float *beta_raw,
                                   const float *A_log, const float *dt_bias,
                                   float scale, float lower_bound,
                                   const int64_t *cu_seqlens, int32_t num_seqs,
                                   int64_t total_tokens, int32_t H, int32_t K, int32_t V,
                                   int32_t chunk_size, kda_dtype_t in_dtype,
                                   const float *initial_state, float *final_state,
                                   void *o, kda_dtype_t o_dtype, void *stream);
/*
 * Streaming device copy of `bytes` bytes from src to dst on `stream`: the
 * library's own read-once / write-once kernel (16-byte non-temporal loads and
 * stores), used as the measured reference for the HBM rate the other kernels
 * are compared with. bytes must be a multiple of 16, src and dst 16-byte
 * aligned and not overlapping (else KDA_ERR_INVALID_ARG); bytes = 0 enqueues
 * nothing.
 */
kda_status_t kda_stream_copy(const void *src, void *dst, size_t bytes, void *stream);
/*
 * Opt-in check of packed offsets (FlashInfer kda_backward page: offsets are
 * validated by one eager synchronisation, the launch path then trusts them).
 * Copies cu_seqlens to the host on `stream`, synchronises that stream and
 * returns KDA_OK if cu[0] == 0, the values never decrease and
 * cu[num_seqs] == total_tokens, else KDA_ERR_INVALID_ARG.
 */
kda_status_t kda_check_cu_seqlens(const int64_t *cu_seqlens, int32_t num_seqs,
                                  int64_t total_tokens, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
