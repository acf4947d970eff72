/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention operator.
 *
 * The operator is the gated delta rule with a diagonal, per-key-channel
 * forget gate ("Kimi Linear" page, sections "Kimi Delta Attention" and
 * "The constrained DPLR form and the chunkwise algorithm"):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,          alpha_t = exp(log_alpha_t) per key channel,
 *
 * with the state S (dk x dv per sequence and head) kept in fp32.  Prefill
 * evaluates it chunkwise (64-token chunks, WY/UT form inside a chunk,
 * recurrent between chunks, as the same page section describes); decode
 * applies one token per sequence.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer owned by the caller; the library
 *    allocates no device memory and keeps no state between calls, so calls
 *    are thread-safe and re-entrant per stream.  KDA_VALUE_SLICE=16, 32 or 64
 *    overrides the number of value columns each state-pass workgroup carries
 *    (by default 16 for at most 64 (sequence, head) pairs, 32 up to 256, else
 *    64; 32 for dk = 64).  With at most 32 state-pass workgroups (for
 *    example four heads of one sequence) and sequences of at least 32 chunks
 *    the prefill runs its state pass sequence-parallel: each sequence is
 *    split into segments that run concurrently from a zero state while also
 *    forming their transition product, a small scan gives every segment its
 *    true initial state, and the segments then form the outputs in parallel;
 *    the workspace size then covers every chunk record.  KDA_SEGMENTS=0 turns
 *    this off and KDA_SEGMENTS=n asks for n segments.  These variables are
 *    read on every call and change scheduling only; results differ at most by
 *    floating-point summation order.
 *  - Layouts are row-major and contiguous.  Tokens are [B, T, H, d] (d
 *    fastest); the recurrent state is [N, H, dk, dv] with dv fastest, rows =
 *    key channels, and the same layout serves initial, final and decode
 *    states.  Data pointers must be 16-byte aligned.
 *  - Supported head dims: dk == dv, and dk in {64, 128}.  q/k/v dtype is
 *    fp32 or bf16; log_alpha and beta are always fp32; out is fp32 or bf16.
 *  - Preconditions not checked on the device: log_alpha finite and <= 0
 *    (any such value: a chunk whose decay ratios would leave the range of the
 *    common single-anchor form is formed in a multi-level form whose factors are
 *    all at most 1; the backward's fp32-input precision degrades in proportion to
 *    the cumulative log decay inside a 64-token chunk past about 100); beta finite;
 *    cu_seqlens non-decreasing with cu_seqlens[0] = 0 and
 *    cu_seqlens[N] = total tokens, and no sequence longer than max_seqlen.
 *    With the environment variable KDA_CHECK=1, kda_chunk_fwd copies
 *    cu_seqlens to the host (synchronising `stream`) and returns
 *    KDA_ERR_INVALID_ARG when one of the cu_seqlens conditions fails.
 *    With bf16 q/k/v the matrix-core
 *    operands are staged in fp16, so |v|, state entries and outputs must
 *    stay below 6.5e4 (larger values give non-finite results, never silent
 *    garbage); q and k are expected L2-normalised per head as in the KDA
 *    layer.  With KDA_CHECK=1 and bf16 inputs, kda_chunk_fwd,
 *    kda_chunk_fwd_noalloc, kda_layer_fwd and kda_chunk_bwd also measure
 *    max|v| and max|init_state| on the device (synchronising `stream`) and,
 *    past 1024, run that call with fp32 matrix-core operands and records
 *    (correct for any finite magnitude; the workspace sizes returned for
 *    bf16 inputs cover it).  kda_layer_fwd with an out_gate and bf16 output
 *    then returns KDA_ERR_UNSUPPORTED: its o passes through fp16 in the
 *    output buffer.  The general DPLR variant has no such switch.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *    and runs asynchronously; results are valid once the stream is
 *    synchronised.  Argument validation is synchronous: on any error no
 *    work is enqueued and a status other than KDA_OK is returned.  No entry
 *    point prints, aborts or throws.
 */
#ifndef KDA_H_
#define KDA_H_

#include <hip/hip_runtime_api.h> /* hipStream_t */
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 } kda_dtype_t;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer, bad aliasing */
    KDA_ERR_UNSUPPORTED = 2, /* a shape or dtype outside the supported set */
    KDA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    KDA_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} kda_status_t;

/* Problem description for the chunked prefill.
 *   batch       dense batch B; must be 1 when cu_seqlens is given
 *   seqlen      tokens per sequence (dense) or total packed tokens (varlen)
 *   num_seqs    0 for a dense batch (N = batch); varlen: N = len(cu_seqlens) - 1
 *               (kda_chunk_fwd treats the call as varlen iff cu_seqlens != NULL;
 *               the workspace query treats the shape as varlen iff num_seqs > 0)
 *   heads, dk, dv, in_dtype (q/k/v), out_dtype (out)
 * Two trailing fields extend the description; zero-initialising them gives the
 * plain per-channel KDA operator with launches sized from seqlen:
 *   max_seqlen  varlen: an upper bound on the longest sequence (host value,
 *               used to size the launch); 0 means "use seqlen"
 *   gate_per_head  0: log_alpha holds one gate per key channel, [.., H, dk]
 *               (KDA); 1: one gate per head shared by all key channels,
 *               [.., H] (the scalar forget gate of Gated DeltaNet, "Kimi
 *               Linear" page, "Background: from the delta rule to gated
 *               DeltaNet") */
typedef struct {
    int32_t batch;
    int64_t seqlen;
    int32_t num_seqs;
    int32_t heads;
    int32_t dk;
    int32_t dv;
    kda_dtype_t in_dtype;
    kda_dtype_t out_dtype;
    int64_t max_seqlen;
    int32_t gate_per_head;
} kda_shape_t;

/* Bytes of scratch device memory kda_chunk_fwd needs for `s` (0 if `s` is
 * invalid).  Any workspace at least this large works; a larger one lets the
 * library keep more chunks per launch. */
size_t kda_chunk_fwd_workspace_size(const kda_shape_t* s);

/* Chunked KDA prefill ("Kimi Linear" page, "The constrained DPLR form and the
 * chunkwise algorithm": 64-token chunks, WY representation, UT transform,
 * recurrent between chunks and parallel inside each).
 *   q, k        [B, T, H, dk]  in_dtype
 *   v           [B, T, H, dv]  in_dtype
 *   log_alpha   [B, T, H, dk]  fp32, natural log of the per-channel gate
 *               ([B, T, H] when s->gate_per_head = 1)
 *   beta        [B, T, H]      fp32
 *   init_state  [N, H, dk, dv] fp32, or NULL for a zero initial state
 *   cu_seqlens  int32 [N+1] device array of packed sequence offsets, or NULL
 *               for a dense batch (then N = B, each sequence T tokens)
 *   out         [B, T, H, dv]  out_dtype; must not alias any input
 *   final_state [N, H, dk, dv] fp32, or NULL; may equal init_state exactly
 *               (in-place continuation) but must not partially overlap it, nor
 *               overlap any other argument
 *   workspace   device scratch of workspace_bytes >= the size above, overlapping
 *               no other argument
 * Sequences of length 0 return final_state = init_state.  One launch holds at
 * most 65535 / N chunks of every sequence (longer sequences run in windows),
 * so N <= 65535, else KDA_ERR_UNSUPPORTED. */
kda_status_t kda_chunk_fwd(const kda_shape_t* s, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, const float* init_state,
                           const int32_t* cu_seqlens, void* out, float* final_state,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* kda_chunk_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, allocation-free serving loops, harnesses that forbid
 * hipMalloc).  Arguments as for kda_chunk_fwd, without the workspace: scratch
 * comes from a static device array of KDA_NOALLOC_SCRATCH_BYTES in the library,
 * one per device it runs on, held until the process ends.  Nothing is allocated
 * (no hipMalloc, hipFree or allocating library call).  The first call on a
 * device looks up that device's array once.  Shapes whose least workspace (the
 * state buffer when final_state is NULL, plus one chunk of records per
 * (sequence, head)) exceeds the array return KDA_ERR_WORKSPACE.  Every call on a
 * device uses that device's one array: calls that overlap in time on one device
 * (other streams, other threads) race and must be serialised by the caller.  The
 * array keeps the last call's contents; no call relies on any part of it
 * starting at zero. */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
kda_status_t kda_chunk_fwd_noalloc(const kda_shape_t* s, const void* q, const void* k, const void* v,
                                   const float* log_alpha, const float* beta, const float* init_state,
                                   const int32_t* cu_seqlens, void* out, float* final_state, hipStream_t stream);

/* General DPLR transition, the form KDA constrains ("Kimi Linear" page, "The
 * constrained DPLR form and the chunkwise algorithm"): a diagonal gate plus a
 * rank-one term whose vectors a and b are independent of the key,
 *
 *     S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,    o_t = S_t^T q_t,
 *
 * where a_t b_t^T acts on the state before the token's decay (b_t^T S_{t-1}).
 * KDA is the case a = beta k, b = alpha (.) k with write key beta k.  Evaluated
 * chunkwise like kda_chunk_fwd (64-token chunks, a UT transform per chunk, an
 * fp32 state between chunks); four gated products per chunk instead of KDA's two.
 *
 * shape: as for kda_chunk_fwd, with dk = dv = 128 and gate_per_head = 0 only
 *   (otherwise KDA_ERR_UNSUPPORTED).
 * q, k, a, b: [.., H, dk] and v [.., H, dv] in shape->in_dtype; k is the write
 *   key (any learning rate folded in); log_alpha fp32 [.., H, dk]; no beta.
 * init_state, cu_seqlens, out, final_state, workspace, stream: as kda_chunk_fwd,
 *   with the same alignment, aliasing and error rules (a and b count as inputs).
 * Preconditions not checked on the device: log_alpha finite and <= 0 (any such
 *   value; diagonal blocks whose single-anchor factors leave their range are
 *   formed in a form with every factor at most 1); a, b and k such that the
 *   state stays bounded; with bf16 inputs the fp16 staging bound of kda_chunk_fwd
 *   on q, k, a, b, v, the state and the outputs. */
size_t kda_dplr_chunk_fwd_workspace_size(const kda_shape_t* s);
kda_status_t kda_dplr_chunk_fwd(const kda_shape_t* s, const void* q, const void* k, const void* v, const void* a,
                                const void* b, const float* log_alpha, const float* init_state,
                                const int32_t* cu_seqlens, void* out, float* final_state, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* One recurrent decode step for `batch` independent sequences ("Kimi Linear"
 * page, "Why linear attention exists": decoding is a recurrent update whose
 * cost does not depend on context length; "Kimi Delta Attention" for the
 * update itself).  Per (sequence, head), with alpha = exp(log_alpha):
 *     S <- Diag(alpha) S;  u = beta (v - S^T k);  S <- S + k u^T;  o = S^T q.
 *   q, k        [batch, H, dk] in_dtype;   v [batch, H, dv] in_dtype
 *   log_alpha   [batch, H, dk] fp32;       beta [batch, H] fp32
 *   state_inout [batch, H, dk, dv] fp32, read and overwritten in place
 *   out         [batch, H, dv] out_dtype
 * No two of state_inout, out and the inputs may overlap (KDA_ERR_INVALID_ARG).
 * batch = 0 does nothing and returns KDA_OK. */
kda_status_t kda_decode_step(int32_t batch, int32_t heads, int32_t dk, int32_t dv,
                             kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                             const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, float* state_inout, void* out, hipStream_t stream);

/* kda_decode_step with one gate per (sequence, head) shared by the key
 * channels: log_alpha is [batch, H] fp32 (the scalar forget gate of Gated
 * DeltaNet, "Kimi Linear" page, "Background: from the delta rule to gated
 * DeltaNet").  Every other argument as for kda_decode_step. */
kda_status_t kda_decode_step_head_gate(int32_t batch, int32_t heads, int32_t dk, int32_t dv,
                                       kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                                       const void* q, const void* k, const void* v, const float* log_alpha,
                                       const float* beta, float* state_inout, void* out, hipStream_t stream);

/* One recurrent step of the general DPLR transition (as kda_dplr_chunk_fwd,
 * "Kimi Linear" page, "The constrained DPLR form and the chunkwise algorithm"):
 * per (sequence, head), with alpha = exp(log_alpha) and w = b^T S read from the
 * state before the token's decay,
 *     S <- Diag(alpha) S - a w^T + k v^T;   o = S^T q.
 * It reads and writes the state once, as kda_decode_step does.
 *   q, k, a, b  [batch, H, dk] in_dtype;   v [batch, H, dv] in_dtype
 *   log_alpha   [batch, H, dk] fp32 (no beta: the learning rate sits in a and k)
 *   state_inout [batch, H, dk, dv] fp32, read and overwritten in place
 *   out         [batch, H, dv] out_dtype
 * dk == dv in {64, 128}.  No two of state_inout, out and the inputs may overlap
 * (KDA_ERR_INVALID_ARG).  batch = 0 does nothing and returns KDA_OK. */
kda_status_t kda_dplr_decode_step(int32_t batch, int32_t heads, int32_t dk, int32_t dv,
                                  kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                                  const void* q, const void* k, const void* v, const void* a, const void* b,
                                  const float* log_alpha, float* state_inout, void* out, hipStream_t stream);

/* Layer prologue and epilogue fused around the operator ("Kimi Linear" page,
 * "Kimi Delta Attention" section): before the recurrence, q and k are scaled
 * to unit L2 norm per head and the per-channel decay is formed from the
 * output of a low-rank projection; after it, each head's output is divided
 * by its RMS and multiplied by a sigmoid gate.  The page fixes neither the map from the projection to the
 * decay nor the constants; this library takes log alpha = -softplus(g) (alpha
 * = sigmoid(-g)) and the epsilons below inside the square roots.
 *   qk_l2norm    1: q and k of every (token, head) are divided by
 *                sqrt(sum over the dk channels of x^2 + l2_eps) before use;
 *                0: used as given
 *   l2_eps       >= 0 (with 0, an all-zero q or k row gives non-finite results)
 *   gate         required, bf16 gate pre-activation g (the projection output),
 *                [.., H, dk], or [.., H] when gate_per_head = 1; it replaces
 *                log_alpha: log alpha = -softplus(g), any finite g.
 *   out_gate     bf16 [.., H, dv] output-gate pre-activation z, or NULL for no
 *                epilogue (the output is then o itself)
 *   norm_weight  fp32 [dv] RMSNorm weight shared by the heads, or NULL (ones)
 *   rms_eps      >= 0: y = o / sqrt(mean over dv of o^2 + rms_eps) * w * sigmoid(z)
 * The pointers are device pointers owned by the caller, 16-byte aligned. */
typedef struct {
    int32_t qk_l2norm;
    float l2_eps;
    const void* gate;
    const void* out_gate;
    const float* norm_weight;
    float rms_eps;
} kda_layer_t;

/* Chunked prefill of the layer: kda_chunk_fwd with the prologue and epilogue
 * of `layer` (log_alpha replaced by layer->gate).  Arguments, layouts and the
 * workspace (kda_chunk_fwd_workspace_size of the same shape) are those of
 * kda_chunk_fwd; `out` holds y.  With an epilogue the state pass first writes
 * o into `out` (fp16 when out_dtype is bf16, so |o| must stay below 6.5e4) and
 * a last pass rewrites it in place as y. */
kda_status_t kda_layer_fwd(const kda_shape_t* s, const kda_layer_t* layer, const void* q, const void* k,
                           const void* v, const float* beta, const float* init_state,
                           const int32_t* cu_seqlens, void* out, float* final_state, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* One decode step of the layer: kda_decode_step with the prologue and epilogue
 * of `layer` (log_alpha replaced by layer->gate, [batch, H, dk] or [batch, H];
 * out_gate [batch, H, dv]); `out` holds y. */
kda_status_t kda_layer_decode_step(int32_t batch, int32_t heads, int32_t dk, int32_t dv, kda_dtype_t in_dtype,
                                   kda_dtype_t out_dtype, int32_t gate_per_head, const kda_layer_t* layer,
                                   const void* q, const void* k, const void* v, const float* beta,
                                   float* state_inout, void* out, hipStream_t stream);

/* Reverse mode of the chunked prefill: the gradients of
 *     L = sum(d_out * out) + sum(d_final_state * final_state)
 * with respect to q, k, v, log_alpha, beta and init_state, through the same
 * chunkwise form ("Kimi Linear" page, "The constrained DPLR form and the
 * chunkwise algorithm"; the page gives the form's cost as a training cost).
 * The forward quantities are recomputed from the inputs (nothing is kept from
 * a forward call).  Shape, dtypes and input layouts as for kda_chunk_fwd
 * (d_out has out_dtype and the layout of out).  The workspace holds one window
 * of chunks per sequence: every chunk when those arrays fit 24 GiB, else the
 * chunks are walked in windows from the last to the first after a forward
 * pass that stores the state entering each window (the environment variable
 * KDA_BWD_WINDOW=n asks for n chunks per window).  A window holds at most
 * 65535 / N chunks, so N <= 65535 (else KDA_ERR_UNSUPPORTED).
 *   d_final_state [N, H, dk, dv] fp32, or NULL (zero)
 *   dq, dk        [B, T, H, dk] fp32;   dv [B, T, H, dv] fp32
 *   dlog_alpha    fp32, the layout of log_alpha
 *   dbeta         [B, T, H] fp32
 *   d_init_state  [N, H, dk, dv] fp32, or NULL (not returned)
 *   workspace     device scratch of workspace_bytes >= kda_chunk_bwd_workspace_size
 * Outputs must not overlap any input or one another, and the workspace must
 * overlap no argument. */
size_t kda_chunk_bwd_workspace_size(const kda_shape_t* s);
kda_status_t kda_chunk_bwd(const kda_shape_t* s, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, const float* init_state,
                           const int32_t* cu_seqlens, const void* d_out, const float* d_final_state, float* dq,
                           float* dk, float* dv, float* dlog_alpha, float* dbeta, float* d_init_state,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* kda_status_string(kda_status_t st);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
