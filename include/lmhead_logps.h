/*
 * lmhead_logps.h -- C ABI of the fused LM-head log-prob and entropy head
 * for AMD Instinct MI355X (gfx950).
 *
 * Per token i with hidden row h_i and target id t_i the head computes, over
 * the whole vocabulary and without ever holding the [tokens, vocab] logits:
 *
 *   z      = W h_i                                  (logits, V values)
 *   lse    = log sum_v exp(z_v)
 *   logp   = z[t_i] - lse
 *   entropy= lse - sum_v softmax(z)_v z_v           (nats)
 *
 * and, for a loss L = sum_i g_logp_i logp_i + g_ent_i entropy_i, the
 * gradients dh = dL/dh and dW = dL/dW through
 *
 *   dz = g_logp (onehot(t) - p) - g_ent p (log p + entropy),  p = softmax(z)
 *   dh_i = W^T dz_i,   dW = sum_i dz_i h_i^T.
 *
 * Definitions follow the pages this library is built from:
 *  - SkyRL issue "[tx] support long sequence", "4. Chunked LM Head": the
 *    cross-entropy of the LM head is computed chunk by chunk so the full
 *    logits tensor is never held (10 GB -> about 300 MB at chunk 512).
 *  - google/tunix pull request #2913, the fused sharded log-prob head: one
 *    pass over a chunk's logits gives the target logit by a one-hot select,
 *    the max and exp-sum once and the entropy from the same exponentials;
 *    the backward forms the logits' cotangent in one elementwise pass over
 *    recomputed logits, and both gradient matmuls read that one cotangent;
 *    a loss that differentiates the entropy adds the entropy term. Ids are
 *    valid iff 0 <= id < vocab.
 *  - google/tunix pull request #2876: the chunk loop over flattened tokens,
 *    int32 targets in, float32 log-probs (and entropies) out, results that
 *    do not depend on the chunk size beyond float32 summation order.
 *
 * Conventions for every entry point
 *  - Pointers are device memory owned by the caller (e.g. allocated by
 *    PyTorch), row-major, 16-byte aligned. bf16 values are passed as their
 *    16-bit patterns (uint16_t).
 *  - Shapes: N >= 0 tokens, H > 0 hidden with H % 64 == 0, 0 < V < 2^31.
 *  - chunk_size > 0 counts flattened tokens. It bounds the backward's
 *    [tokens, vocab]-shaped transient: the logits cotangent the backward
 *    holds at any time is at most one float32 [chunk_size, V] tensor in bytes
 *    (it is kept as two bf16 buffers of a block of tokens x vocabulary, the
 *    next block's formed while the current one's is used). The backward
 *    workspace also holds a bf16 transpose of the hidden states
 *    (input-sized), a copy of W's last V % 64 rows and 32 bytes of tile
 *    counters per block (reset by every call). The forward holds no
 *    [tokens, vocab] transient at all. Per-token forward results do not depend on
 *    chunk_size; gradients depend on it only through float32 summation order.
 *  - Targets outside [0, V) (-1 included) mask the token: its logp, entropy
 *    and lse are written as 0, its dh row is written as 0 and it adds nothing
 *    to dW, whatever its hidden row holds (NaN and inf included). They are
 *    not errors.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    default stream). The library never synchronises the device, allocates
 *    no device memory and keeps no state between calls: distinct workspaces
 *    on distinct streams may be used from several threads at once (the
 *    optional tracing at the end of this header is the one exception).
 *  - Outputs are overwritten in full (dW is not accumulated into).
 *  - Non-finite logits in unmasked rows (they arise only from non-finite W
 *    or hidden values; tunix #2913 checks its scoring on inf, -inf and NaN
 *    logits and on a row of no finite logit) follow IEEE evaluation of the
 *    definitions above, the log-sum-exp shifted by the row max when that max
 *    is finite and by 0 otherwise: a -inf entry drops out of lse and a -inf
 *    target gives logp = -inf, while the entropy's p (z - lse) = 0 * -inf
 *    makes that row's entropy NaN; a +inf entry (and no NaN) gives
 *    lse = +inf, logp = -inf (NaN when the target is the +inf entry) and a
 *    NaN entropy; any NaN entry makes the row's three values NaN; a row of
 *    no finite logit has lse = -inf and NaN logp and entropy. Gradients
 *    follow the same arithmetic with two readings in the cotangent: the
 *    entropy term is formed only for tokens with a nonzero g_ent (the
 *    one-pass g_logp (onehot - p) of a loss that stops the entropy's
 *    gradient, tunix #2913), and an entry whose probability is 0 gets no
 *    probability term. So with only log-prob cotangents a -inf entry's
 *    cotangent is g_logp at its targets and 0 elsewhere and the rest of the
 *    row's cotangent is that of the vocabulary without it; the two gradient
 *    products stay IEEE (0 times the -inf table entry is NaN in dh). A +inf
 *    or NaN entry, or a nonzero g_ent on a NaN entropy, makes the cotangent
 *    of that row NaN where the probability is not 0. Masked rows are 0
 *    whatever their hidden row holds.
 *  - Return value: LMH_OK (0) or a negative LMH_ERR_* code. Argument checks
 *    run on the host before anything is enqueued, so a failing call enqueues
 *    nothing. lmhead_logps_last_error() gives a thread-local message for the
 *    last failing call of the calling thread.
 */
#ifndef LMHEAD_LOGPS_H_
#define LMHEAD_LOGPS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LMH_OK 0
#define LMH_ERR_NULL (-1)        /* a required pointer is NULL */
#define LMH_ERR_SHAPE (-2)       /* N < 0, H <= 0, V <= 0 or V >= 2^31 */
#define LMH_ERR_CHUNK (-3)       /* chunk_size <= 0 */
#define LMH_ERR_WORKSPACE (-4)   /* workspace smaller than the queried size */
#define LMH_ERR_ARGS (-5)        /* g_ent given without entropy; bad temperature */
#define LMH_ERR_UNSUPPORTED (-6) /* H % 64 != 0, a misaligned pointer, or a backward with N or V > 2^23 - 256 */
#define LMH_ERR_HIP (-7)         /* a HIP call or kernel launch failed */

/*
 * Bytes of device workspace a call needs. with_backward = LMH_WS_FWD (0)
 * sizes the forward only; LMH_WS_BWD (1) sizes a workspace that serves both
 * the forward and the float32-gradient backward (one buffer may be reused
 * for both calls when they run in stream order); LMH_WS_BWD_BF16 (2) sizes
 * one that also serves lmhead_logps_bwd_bf16. Pure host computation, no
 * device call. Errors: LMH_ERR_NULL (bytes_out), LMH_ERR_SHAPE,
 * LMH_ERR_CHUNK, LMH_ERR_ARGS (with_backward not 0, 1 or 2),
 * LMH_ERR_UNSUPPORTED (a backward with N or V above 2^23 - 256: the backward
 * addresses 256-row tiles of its transposed operands with 32-bit offsets).
 */
#define LMH_WS_FWD 0
#define LMH_WS_BWD 1
#define LMH_WS_BWD_BF16 2
int lmhead_logps_workspace_bytes(int64_t N, int64_t H, int64_t V, int64_t chunk_size,
                                 int with_backward, size_t* bytes_out);

/*
 * Forward: logp, entropy and lse per token (SkyRL "4. Chunked LM Head";
 * tunix #2913 one-pass scoring of logits).
 *   hidden   bf16 [N, H]   token hidden states
 *   W        bf16 [V, H]   output embedding (vocabulary) table
 *   targets  int32 [N]     target ids; outside [0, V) masks the token
 *   logp     f32 [N]       out: z[t] - lse, 0 when masked
 *   entropy  f32 [N]       out, or NULL when not requested; 0 when masked
 *   lse      f32 [N]       out: log-sum-exp of the logits, 0 when masked
 *   workspace / workspace_bytes: device scratch of at least
 *            lmhead_logps_workspace_bytes(N, H, V, chunk_size, 0) bytes;
 *            its contents on entry are ignored.
 * Errors: LMH_ERR_NULL (hidden, W, targets, logp, lse, or workspace when
 * N > 0), LMH_ERR_SHAPE, LMH_ERR_CHUNK, LMH_ERR_WORKSPACE, LMH_ERR_UNSUPPORTED,
 * LMH_ERR_HIP. N = 0 enqueues nothing and returns LMH_OK.
 */
int lmhead_logps_fwd(const uint16_t* hidden, const uint16_t* W, const int32_t* targets,
                     int64_t N, int64_t H, int64_t V, int64_t chunk_size,
                     float* logp, float* entropy, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward: dh and dW of L = sum_i g_logp_i logp_i + g_ent_i entropy_i
 * (tunix #2913: the cotangent of the recomputed logits in one elementwise
 * pass, read by both gradient matmuls; the entropy term when the entropy is
 * differentiated).
 *   hidden, W, targets, N, H, V, chunk_size: as for the forward
 *   lse      f32 [N]       the forward's lse output (required)
 *   entropy  f32 [N]       the forward's entropy output; required iff g_ent
 *   g_logp   f32 [N]       cotangent of logp, or NULL for all zeros
 *   g_ent    f32 [N]       cotangent of entropy, or NULL for all zeros
 *   dh       f32 [N, H]    out, overwritten; masked rows are 0
 *   dW       f32 [V, H]    out, overwritten (not accumulated into)
 *   workspace: at least lmhead_logps_workspace_bytes(..., 1) bytes.
 * Errors: LMH_ERR_NULL, LMH_ERR_SHAPE, LMH_ERR_CHUNK, LMH_ERR_WORKSPACE,
 * LMH_ERR_ARGS (g_ent without entropy), LMH_ERR_UNSUPPORTED (including N or V
 * above 2^23 - 256), LMH_ERR_HIP.
 * N = 0 writes dW = 0 and returns LMH_OK.
 */
int lmhead_logps_bwd(const uint16_t* hidden, const uint16_t* W, const int32_t* targets,
                     int64_t N, int64_t H, int64_t V, int64_t chunk_size,
                     const float* lse, const float* entropy,
                     const float* g_logp, const float* g_ent,
                     float* dh, float* dW,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tempered head (google/tunix pull request #2913 runs its head at
 * temperatures 1 and 0.7): the same two calls scoring the tempered logits
 * z / T. logp, entropy and lse are those of softmax(z / T) (lse of z / T);
 * the backward's cotangent of the tempered logits is divided by T before
 * both gradient matmuls, so dh and dW are gradients with respect to the
 * untempered hidden and W. The backward needs the tempered forward's lse and
 * entropy and the same T. temperature must be finite and > 0 with 1 / T
 * finite in float32, otherwise LMH_ERR_ARGS; all other arguments, layouts, ownership and errors are those
 * of lmhead_logps_fwd / lmhead_logps_bwd, which are these calls at T = 1
 * (bit for bit).
 */
int lmhead_logps_fwd_temp(const uint16_t* hidden, const uint16_t* W, const int32_t* targets,
                          int64_t N, int64_t H, int64_t V, int64_t chunk_size, float temperature,
                          float* logp, float* entropy, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);
int lmhead_logps_bwd_temp(const uint16_t* hidden, const uint16_t* W, const int32_t* targets,
                          int64_t N, int64_t H, int64_t V, int64_t chunk_size, float temperature,
                          const float* lse, const float* entropy,
                          const float* g_logp, const float* g_ent,
                          float* dh, float* dW,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward that adds into the caller's gradient buffers (a trainer's
 * float32 weight-gradient and activation-gradient accumulators; tunix #2913
 * hands the head's gradients to the trainer's own accumulation). The same
 * computation as lmhead_logps_bwd_temp, with
 *   flags & LMH_BWD_ACCUMULATE_DH: dh += gradient (masked rows unchanged)
 *                                   instead of dh = gradient;
 *   flags & LMH_BWD_ACCUMULATE_DW: dW += gradient instead of dW = gradient
 *                                   (N = 0 then leaves dW unchanged).
 * The added values are summed in the same fixed block order as the
 * overwriting call, then added to the buffer's previous contents block by
 * block: deterministic, equal to "previous + gradient" up to float32
 * summation order. Unknown flag bits: LMH_ERR_ARGS. Everything else is that
 * of lmhead_logps_bwd_temp (temperature 1 for the untempered head).
 */
#define LMH_BWD_ACCUMULATE_DH 1u
#define LMH_BWD_ACCUMULATE_DW 2u
int lmhead_logps_bwd_ex(const uint16_t* hidden, const uint16_t* W, const int32_t* targets,
                        int64_t N, int64_t H, int64_t V, int64_t chunk_size, float temperature,
                        const float* lse, const float* entropy,
                        const float* g_logp, const float* g_ent,
                        float* dh, float* dW, unsigned flags,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward writing bf16 gradients (a trainer whose parameters and
 * activations are bf16 takes the head's gradients in their own dtype;
 * tunix #2913 hands the head's gradients to the trainer's own
 * accumulation). The computation of lmhead_logps_bwd_ex, with
 *   dh  bf16 [N, H]   out (masked rows 0), or added into with
 *                     LMH_BWD_ACCUMULATE_DH (masked rows unchanged)
 *   dW  bf16 [V, H]   out, or added into with LMH_BWD_ACCUMULATE_DW
 * both 16-byte aligned. Each gradient element is summed over the blocks in
 * float32 inside the workspace, in the same order as the float32 backward,
 * and rounded to bf16 (nearest even) once, when its last block is added: the
 * result is the float32 backward's rounded to bf16, bit for bit (with an
 * ACCUMULATE flag, the previous bf16 value widened to float32 is the sum's
 * starting value). Workspace: lmhead_logps_workspace_bytes(...,
 * LMH_WS_BWD_BF16) bytes, the float32 backward's plus float32 accumulators
 * of min(N, V) x H elements (the smaller gradient, summed over the whole
 * call) and of one block's rows of the other. Everything else (arguments,
 * errors, N = 0, stream semantics) is that of lmhead_logps_bwd_ex.
 */
int lmhead_logps_bwd_bf16(const uint16_t* hidden, const uint16_t* W, const int32_t* targets,
                          int64_t N, int64_t H, int64_t V, int64_t chunk_size, float temperature,
                          const float* lse, const float* entropy,
                          const float* g_logp, const float* g_ent,
                          uint16_t* dh, uint16_t* dW, unsigned flags,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Vocabulary shards (tunix #2913's head runs sharded, its vocabulary table
 * split across devices, the per-token (max, exp-sum) partials combined across
 * shards; the same log-sum-exp combination as blockwise attention's, palingenesis
 * guide "Long Sequences (SeCO)"). A shard is the rows [vocab_offset,
 * vocab_offset + V_shard) of a vocabulary of V_total ids; W_shard is bf16
 * [V_shard, H]; targets are global ids (valid iff 0 <= t < V_total).
 *
 * lmhead_logps_fwd_shard: writes, per token, the shard's partial record
 *   partial f32 [N][4] (16-byte aligned): (m, s1, s2, zt) with m the max of
 *   the shard's tempered logits in base 2 (log2(e) z / T), s1 = sum 2^(x - m),
 *   s2 = sum 2^(x - m) (x - m) over x = log2(e) z / T, zt the untempered
 *   target logit when the target lies in the shard and 0 otherwise. The
 *   workspace is lmhead_logps_workspace_bytes(N, H, V_shard, chunk_size, 0).
 * lmhead_logps_merge_shards: merges P records per token in shard order,
 *   partials f32 [P][N][4], into logp / entropy (or NULL) / lse of the whole
 *   vocabulary, exactly what lmhead_logps_fwd_temp writes up to float32
 *   rounding (masked tokens 0). Needs no workspace.
 * lmhead_logps_bwd_shard: the shard's part of the backward given the merged
 *   lse / entropy: dW_shard f32 [V_shard, H] and the shard's contribution to
 *   dh (flags as for lmhead_logps_bwd_ex; on one device, the first shard
 *   overwrites dh and the others add with LMH_BWD_ACCUMULATE_DH). Workspace:
 *   lmhead_logps_workspace_bytes(N, H, V_shard, chunk_size, 1).
 * Errors as for the whole-table calls, plus LMH_ERR_SHAPE when the shard does
 * not lie in [0, V_total) or P is not in [1, 65536].
 */
int lmhead_logps_fwd_shard(const uint16_t* hidden, const uint16_t* W_shard, const int32_t* targets,
                           int64_t N, int64_t H, int64_t V_shard, int64_t vocab_offset, int64_t V_total,
                           int64_t chunk_size, float temperature, float* partial,
                           void* workspace, size_t workspace_bytes, void* stream);
int lmhead_logps_merge_shards(const float* partials, int64_t P, const int32_t* targets, int64_t N,
                              int64_t V_total, float temperature,
                              float* logp, float* entropy, float* lse, void* stream);
int lmhead_logps_bwd_shard(const uint16_t* hidden, const uint16_t* W_shard, const int32_t* targets,
                           int64_t N, int64_t H, int64_t V_shard, int64_t vocab_offset, int64_t V_total,
                           int64_t chunk_size, float temperature,
                           const float* lse, const float* entropy,
                           const float* g_logp, const float* g_ent,
                           float* dh, float* dW_shard, unsigned flags,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). The same computation and results
 * as lmhead_logps_fwd_temp (bit for bit); its scratch (the vocabulary-split
 * partial records) lives in a fixed device array of
 * LMH_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends. A call fits iff lmhead_logps_workspace_bytes(N, H, V,
 * chunk_size, 0) <= LMH_NOALLOC_SCRATCH_BYTES (about 300,000 tokens at a
 * 152k vocabulary); larger calls fail with LMH_ERR_WORKSPACE and enqueue
 * nothing. Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (several streams or threads at once) race and must not be made;
 * calls in stream order are safe (each call writes every record it reads).
 * The work runs on the stream's device (the current device for the NULL
 * stream); the first call there looks the array's address up with that
 * device current and restores the caller's (set-up, no allocation). With
 * the library's tracing on (a measurement facility, off by default), every
 * launch also records two HIP events, which the tracing creates on first
 * use. Errors: as for lmhead_logps_fwd_temp, plus
 * LMH_ERR_WORKSPACE as above and LMH_ERR_HIP if the address lookup fails.
 */
#define LMH_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
int lmhead_logps_fwd_noalloc(const uint16_t* hidden, const uint16_t* W, const int32_t* targets,
                             int64_t N, int64_t H, int64_t V, int64_t chunk_size, float temperature,
                             float* logp, float* entropy, float* lse, void* stream);

/* Thread-local message of the calling thread's last failing call ("" if none). */
const char* lmhead_logps_last_error(void);

/* Library version string. */
const char* lmhead_logps_version(void);

/*
 * Tracing (measurement only; not needed to use the head). While enabled,
 * every kernel launch of the library is bracketed by two HIP events on the
 * stream it runs on and tagged with its algorithmic work. Kernel ids:
 *   0 fwd_stats_kernel  (forward logits tiles + running statistics)
 *   1 fwd_merge_kernel  (split merge)
 *   2 bwd_step_kernel   (dh and dW GEMMs of one block + the logits recompute
 *                        and cotangent of the next block)
 *   3 transpose_kernel  (bf16 transpose of the hidden states)
 *   4 fill_zero_kernel
 *   5 pad_rows_kernel   (W's last V % 64 rows, zero-padded to 64)
 *   6 bwd_step_bf16_kernel (bwd_step_kernel writing bf16 gradients)
 * lmhead_logps_trace_enable(on) clears the totals and starts (on != 0) or
 * stops recording. lmhead_logps_trace_read(kernel, ...) waits for the
 * recorded launches to finish and returns, for that kernel, the launch
 * count, the summed duration in ms and the summed algorithmic flops and
 * bytes. Algorithmic flops are the credited work: 2 H per (token, vocabulary)
 * element for the forward's logits and for each of the backward's two
 * gradient GEMMs; the backward's recompute of the logits (another 2 H per
 * element) is executed but not counted. This state is process-wide;
 * enabling it adds two event records per
 * launch. Errors: LMH_ERR_ARGS (unknown kernel id), LMH_ERR_NULL.
 * lmhead_logps_trace_kernel_name returns NULL for an unknown id.
 */
int lmhead_logps_trace_enable(int on);
int lmhead_logps_trace_read(int kernel, int64_t* launches, double* total_ms, double* flops,
                            double* bytes);
const char* lmhead_logps_trace_kernel_name(int kernel);

#ifdef __cplusplus
}
#endif

#endif /* LMHEAD_LOGPS_H_ */
