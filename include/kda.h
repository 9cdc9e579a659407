/*
 * kda.h - Kimi Delta Attention (KDA) forward kernels for AMD MI355X (gfx950).
 *
 * KDA is the channel-wise gated delta rule.  Per head, a d_k x d_v fast-weight
 * state evolves token by token as
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,          alpha_t = exp(g_t)  (one factor per key channel)
 *
 * with the decay applied before the delta-rule correction and the output read
 * from the updated state.  Sources: the "Kimi Linear" notes (docsaid.org),
 * section "KDA: Splitting the Decay Across Channels"; the greeksharifa.github.io
 * summary of the Kimi Linear report, section 3 "Kimi Delta Attention".  No query
 * scale is applied (none appears on those pages); callers pre-scale q.
 *
 * Two entry points cover the two ways the pages say the operator runs
 * (greeksharifa summary, section 6.3 "Complexity Analysis"): prompt processing
 * uses the chunkwise algorithm (kda_prefill) and generation uses the recurrent
 * single-token update (kda_decode_step).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or retains device memory.
 *  - Layouts are contiguous and token-major: q, k, g are [tokens, H, Dk];
 *    v and o are [tokens, H, Dv]; beta is [tokens, H].  States are
 *    [N, H, Dk, Dv] float32 with Dv contiguous.
 *  - in_dtype selects the element type of q, k, v (KDA_BF16 or KDA_F32);
 *    g, beta and the states are always float32.  out_dtype selects o.
 *  - g is the log-decay: finite and <= 0 (alpha in (0, 1]).  Values are not
 *    checked; NaN/Inf propagate.  g > 0 is outside the supported domain.
 *  - Work is enqueued asynchronously on `stream` (NULL = the default stream).
 *    Argument errors are detected on the host, before anything is enqueued,
 *    and are returned synchronously.  A launch failure returns KDA_ERR_HIP.
 *  - No C++ exception crosses this interface.
 *  - Pointers must be 16-byte aligned.
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
  KDA_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad cu_seqlens, misaligned */
  KDA_ERR_UNSUPPORTED = 2, /* head size or chunk size not built */
  KDA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  KDA_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} kda_status;

typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* kda_status_string(kda_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int kda_version(void);

/*
 * Workspace bytes that kda_prefill needs for this problem.  Arguments have the
 * same meaning as in kda_prefill.  Returns 0 and writes nothing to *bytes on
 * an argument error (the status says which).
 *
 * The prefill runs in segments, each covering the same range of local chunks
 * of every sequence.  The workspace holds a per-segment slot table (varlen
 * only), the intra-chunk operands of one segment (144.5 KB per chunk and head
 * at Dk = Dv = 128, C = 64; about 160 MiB per segment when there are few
 * (sequence, head) pairs, up to 8 GiB otherwise) and, when there is more
 * than one segment, the fp32 state carried between them (num_seqs * H * Dk *
 * Dv * 4 bytes).  So the size is bounded for any sequence length.  The size
 * depends only on the arguments: kda_prefill_ex with non-default options
 * needs kda_prefill_workspace_size_ex with the same options.
 */
kda_status kda_prefill_workspace_size(int B, int T, int H, int Dk, int Dv,
                                      int num_seqs,
                                      const int32_t* cu_seqlens_host,
                                      int chunk_size, kda_dtype in_dtype,
                                      size_t* bytes);

/*
 * Chunked KDA forward pass (prompt processing).
 *
 * Computes o for every token and, optionally, the final state of every
 * sequence, exactly as the token-by-token recurrence above, using the
 * chunkwise algorithm of the Kimi Linear report: within each chunk of
 * `chunk_size` tokens the work is parallel (WY representation of the rank-1
 * updates, UT transform solved by forward substitution, causally masked
 * intra-chunk term); between chunks the state is carried recurrently
 * (greeksharifa summary, section 3.1 "Hardware-Efficient Chunkwise
 * Algorithm"; zeroshot.it.com deep-dive, section 4 "Chunking and Kernels").
 *
 * Sequences:
 *   - cu_seqlens == NULL: B sequences of T tokens each, tensors [B, T, H, *].
 *     num_seqs must equal B.
 *   - cu_seqlens != NULL (varlen packing): B must be 1; the tensors hold
 *     T = cu_seqlens_host[num_seqs] tokens; sequence n is the token range
 *     [cu_seqlens[n], cu_seqlens[n+1]).  Both the device copy (read by the
 *     kernels) and an identical host copy (validated, sizes the launch) are
 *     required.  Values must be non-decreasing from 0 and end at T.  Empty
 *     sequences are allowed (their final state equals their initial state).
 *   Chunks start at each sequence start and never cross sequences; the last
 *   chunk of a sequence may be shorter than chunk_size.
 *
 * Arguments:
 *   q, k          [B*T, H, Dk]  in_dtype
 *   v             [B*T, H, Dv]  in_dtype
 *   g             [B*T, H, Dk]  float32 log-decay (<= 0)
 *   beta          [B*T, H]      float32
 *   o             [B*T, H, Dv]  out_dtype (written)
 *   initial_state [num_seqs, H, Dk, Dv] float32, or NULL for zeros
 *   final_state   [num_seqs, H, Dk, Dv] float32, or NULL (not written);
 *                 may alias initial_state
 *   Dk, Dv        head sizes; supported: Dk == Dv in {64, 128}
 *   chunk_size    16, 32 or 64
 *   workspace     device buffer of at least kda_prefill_workspace_size bytes,
 *                 256-byte aligned; contents need not be initialised and are
 *                 garbage afterwards.  Must not be shared with a call that
 *                 runs concurrently.
 */
kda_status kda_prefill(const void* q, const void* k, const void* v,
                       const float* g, const float* beta, void* o,
                       const float* initial_state, float* final_state,
                       const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                       int B, int T, int H, int Dk, int Dv, int num_seqs,
                       int chunk_size, kda_dtype in_dtype, kda_dtype out_dtype,
                       void* workspace, size_t workspace_bytes,
                       void* stream /* hipStream_t */);

/*
 * kda_prefill for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops that forbid allocation, and harnesses that
 * forbid hipMalloc.  Same arguments and results as kda_prefill, without the
 * workspace: the intermediate data lives in a static device array of
 * KDA_PREFILL_NOALLOC_SCRATCH_BYTES (128 MiB) that each GPU the library runs
 * on holds until the process ends.  The call allocates and frees nothing.
 *
 * The prefill runs in segments whose whole workspace fits that array (the
 * segments are shorter than kda_prefill's when the problem is large, so the
 * call may take longer; results are the same).  A problem that does not fit
 * even with one-chunk segments -- the fp32 state carried between segments,
 * num_seqs * H * Dk * Dv * 4 bytes, plus one chunk of every sequence's
 * operands -- returns KDA_ERR_WORKSPACE before anything is enqueued.
 *
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (other streams, other host threads) race and corrupt each
 * other's results.  Serialise them.  Nothing in the array needs clearing
 * between calls.
 */
#define KDA_PREFILL_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

kda_status kda_prefill_noalloc(const void* q, const void* k, const void* v,
                               const float* g, const float* beta, void* o,
                               const float* initial_state, float* final_state,
                               const int32_t* cu_seqlens,
                               const int32_t* cu_seqlens_host, int B, int T,
                               int H, int Dk, int Dv, int num_seqs,
                               int chunk_size, kda_dtype in_dtype,
                               kda_dtype out_dtype,
                               void* stream /* hipStream_t */);

/*
 * Choices kda_prefill normally makes itself, for callers that tune the
 * launch or need to exercise a particular configuration.  Every field left
 * at zero keeps the automatic choice; results are identical for every
 * setting (they change only how the work is split).
 *   segment_chunks  local chunks of every sequence per segment (>= 1); each
 *                   segment is one intra-chunk pass and one carry pass, and
 *                   the state is carried between segments in the workspace
 *   segment_bytes   operand budget of one segment in bytes (segment_chunks
 *                   then follows from it); ignored when segment_chunks is set
 *   value_block     value columns per workgroup of the carry pass: 16 or 32
 * Invalid values (negative, value_block not 0/16/32) give
 * KDA_ERR_INVALID_ARG.
 */
typedef struct {
  int segment_chunks;
  size_t segment_bytes;
  int value_block;
} kda_prefill_options;

/* The three chunked forward forms that share the prefill kernels. */
typedef enum {
  KDA_FORM_KDA = 0,   /* kda_prefill */
  KDA_FORM_GDN = 1,   /* gdn_prefill: g is [B*T, H] */
  KDA_FORM_LAYER = 2  /* kda_prefill_layer: inputs before their activations */
} kda_prefill_form;

/*
 * kda_prefill, gdn_prefill or kda_prefill_layer (selected by `form`) with
 * explicit options (NULL: automatic, the same as the plain entry points).
 * `layer` (a kda_layer_params*, declared below) is read for KDA_FORM_LAYER
 * only, and may be NULL there as in kda_prefill_layer.  The workspace must be
 * sized by kda_prefill_workspace_size_ex with the same form, layer and
 * options.  An unknown form gives KDA_ERR_INVALID_ARG.
 */
kda_status kda_prefill_workspace_size_ex(int form, int B, int T, int H, int Dk,
                                         int Dv, int num_seqs,
                                         const int32_t* cu_seqlens_host,
                                         int chunk_size, kda_dtype in_dtype,
                                         const void* layer,
                                         const kda_prefill_options* options,
                                         size_t* bytes);

kda_status kda_prefill_ex(int form, const void* q, const void* k, const void* v,
                          const float* g, const float* beta, const void* layer,
                          void* o, const float* initial_state,
                          float* final_state, const int32_t* cu_seqlens,
                          const int32_t* cu_seqlens_host, int B, int T, int H,
                          int Dk, int Dv, int num_seqs, int chunk_size,
                          kda_dtype in_dtype, kda_dtype out_dtype,
                          const kda_prefill_options* options, void* workspace,
                          size_t workspace_bytes, void* stream /* hipStream_t */);

/*
 * One recurrent KDA step for N independent sequences (generation).
 *
 * For every sequence n and head h, with one new token (q, k, v, g, beta):
 *   S <- Diag(exp(g)) S;  u = beta (v - S^T k);  S <- S + k u^T;  o = S^T q
 * (greeksharifa summary, section 3 and section 6.3: generation uses the
 * recurrent update).  The state is read and written in place.
 *
 * Arguments:
 *   q, k   [N, H, Dk]  in_dtype
 *   v      [N, H, Dv]  in_dtype
 *   g      [N, H, Dk]  float32 log-decay (<= 0)
 *   beta   [N, H]      float32
 *   state  [N, H, Dk, Dv] float32, updated in place
 *   o      [N, H, Dv]  out_dtype (written)
 *   Dk, Dv supported: Dk == Dv in {64, 128}
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v,
                           const float* g, const float* beta, float* state,
                           void* o, int N, int H, int Dk, int Dv,
                           kda_dtype in_dtype, kda_dtype out_dtype,
                           void* stream /* hipStream_t */);

/*
 * Gated DeltaNet: the scalar-decay special case of KDA, with one log-decay
 * per token and head shared by all key channels,
 *
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *
 * (zeroshot.it.com deep-dive, section 2.3; the docsaid.org "Kimi Linear"
 * notes, section "KDA: Splitting the Decay Across Channels", give it as the
 * form KDA refines).  It equals kda_prefill / kda_decode_step with g
 * broadcast over the key channels, runs through the same kernels, and reads
 * Dk times fewer decay values.
 *
 * Arguments and behaviour are those of kda_prefill / kda_decode_step except:
 *   g   [B*T, H] (prefill) or [N, H] (decode) float32 log-decay (<= 0)
 * kda_prefill_workspace_size gives the workspace size for gdn_prefill too.
 */
kda_status gdn_prefill(const void* q, const void* k, const void* v,
                       const float* g, const float* beta, void* o,
                       const float* initial_state, float* final_state,
                       const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                       int B, int T, int H, int Dk, int Dv, int num_seqs,
                       int chunk_size, kda_dtype in_dtype, kda_dtype out_dtype,
                       void* workspace, size_t workspace_bytes,
                       void* stream /* hipStream_t */);

kda_status gdn_decode_step(const void* q, const void* k, const void* v,
                           const float* g, const float* beta, float* state,
                           void* o, int N, int H, int Dk, int Dv,
                           kda_dtype in_dtype, kda_dtype out_dtype,
                           void* stream /* hipStream_t */);

/*
 * The KDA layer's elementwise work fused around the recurrence (the docsaid.org
 * "Kimi Linear" notes, section "Other Components"; the greeksharifa.github.io
 * summary, section 4 "Model Architecture").  The inputs are the projections
 * before their activations:
 *
 *   q = L2norm(Swish(conv_q(q_pre))),  k = L2norm(Swish(conv_k(k_pre)))
 *   v = Swish(conv_v(v_pre)),          beta = sigmoid(beta_logit)
 *
 * per (token, head), with Swish(x) = x * sigmoid(x) and L2norm(x) =
 * x / max(|x|_2, 1e-12).  conv_x is the short convolution: causal and
 * depthwise over the tokens of each sequence, of width W (1..4), no bias:
 *
 *   conv(x)[t, h, c] = sum_{i<W} weight[h, c, i] * x[t - (W-1) + i, h, c]
 *
 * where inputs before the sequence's first token come from the carried
 * state (row (W-1) + (s - first token); zeros when the state is NULL).  With
 * conv_width = 0 the convolution is skipped.  The recurrence then runs as in
 * kda_prefill / kda_decode_step.  When gate is not NULL the output is
 *
 *   y[t, h, c] = o[t, h, c] / sqrt(mean_c' o[t, h, c']^2 + norm_eps)
 *                * norm_weight[c] * sigmoid(gate[t, h, c])
 *
 * (head-wise RMSNorm with a per-channel weight shared by the heads, times the
 * output gate); when gate is NULL, o itself is written and norm_weight and
 * norm_eps are ignored.  The final states are those of the recurrence.
 */
typedef struct {
  const void* gate;           /* [tokens, H, Dv] in_dtype, or NULL: no epilogue */
  const float* norm_weight;   /* [Dv] float32; required with gate */
  float norm_eps;             /* finite, >= 0 */
  int conv_width;             /* 0: no short convolution; else 1..4 */
  const float* conv_weight[3]; /* q, k, v: [H, D, conv_width] float32 (with conv) */
  /* Carried convolution inputs of q, k, v: [num_seqs (or N), H, conv_width-1,
   * D] in_dtype, row conv_width-2 the most recent.  conv_state_in NULL: zeros.
   * conv_state_out receives the last conv_width-1 inputs of each sequence
   * after the call (NULL: not written); it may alias conv_state_in. */
  const void* conv_state_in[3];
  void* conv_state_out[3];
} kda_layer_params;

/*
 * Workspace bytes of kda_prefill_layer (layer may be NULL: no epilogue).  With
 * a gate the workspace also holds one segment's raw fp32 output (chunk * Dv *
 * 4 bytes per chunk and head), because the norm spans value columns that the
 * inter-chunk pass computes in separate workgroups.
 */
kda_status kda_prefill_layer_workspace_size(int B, int T, int H, int Dk, int Dv,
                                            int num_seqs,
                                            const int32_t* cu_seqlens_host,
                                            int chunk_size, kda_dtype in_dtype,
                                            const kda_layer_params* layer,
                                            size_t* bytes);

/*
 * Arguments are those of kda_prefill / kda_decode_step, plus:
 *   q_pre, k_pre, v_pre  as q, k, v (in_dtype)
 *   beta_logit  [tokens, H] float32 (sigmoid applied inside)
 *   layer       gate, RMSNorm weight and eps, short convolution; NULL means
 *               no convolution and no epilogue (the prologue still runs)
 * For kda_decode_step_layer the convolution states are [N, H, conv_width-1,
 * D]: one step reads conv_state_in and writes the shifted inputs (the new
 * token last) to conv_state_out, which is normally the same buffer.
 */
kda_status kda_prefill_layer(const void* q_pre, const void* k_pre,
                             const void* v_pre, const float* g,
                             const float* beta_logit,
                             const kda_layer_params* layer, void* o,
                             const float* initial_state, float* final_state,
                             const int32_t* cu_seqlens,
                             const int32_t* cu_seqlens_host, int B, int T,
                             int H, int Dk, int Dv, int num_seqs,
                             int chunk_size, kda_dtype in_dtype,
                             kda_dtype out_dtype, void* workspace,
                             size_t workspace_bytes,
                             void* stream /* hipStream_t */);

kda_status kda_decode_step_layer(const void* q_pre, const void* k_pre,
                                 const void* v_pre, const float* g,
                                 const float* beta_logit,
                                 const kda_layer_params* layer, float* state,
                                 void* o, int N, int H, int Dk, int Dv,
                                 kda_dtype in_dtype, kda_dtype out_dtype,
                                 void* stream /* hipStream_t */);

/*
 * Backward pass of kda_prefill: the gradients of
 *
 *     L = sum(d_o * o) + sum(d_final_state * final_state)
 *
 * with respect to q, k, v, g, beta and the initial state, for the same
 * inputs and sequence description as the forward call (the pages say the
 * chunkwise form serves training: greeksharifa summary, sections 3.1 and
 * 6.3; the gradients are the chain rule through the chunk form of the
 * recurrence).  The forward pass is recomputed inside; o is not needed.
 * Arithmetic is fp32; the decay enters every intra-chunk pair through the
 * exact exponent of its difference, so any decay strength is handled.
 *
 * Arguments (others as in kda_prefill):
 *   d_o            [B*T, H, Dv] float32
 *   d_final_state  [num_seqs, H, Dk, Dv] float32, or NULL (zero)
 *   dq, dk, dg     [B*T, H, Dk] float32 (written)
 *   dv             [B*T, H, Dv] float32 (written)
 *   dbeta          [B*T, H] float32 (written)
 *   d_initial_state [num_seqs, H, Dk, Dv] float32, or NULL (not written)
 *   workspace      at least kda_backward_workspace_size bytes, 256-byte
 *                  aligned.  The backward runs in segments of local chunks
 *                  of every sequence, as kda_prefill does: a forward sweep
 *                  keeps only the state entering each segment, and the
 *                  backward sweep (last segment first) recomputes one
 *                  segment's fp32 intermediates (about 737 KB per chunk and
 *                  head at Dk = Dv = 128, C = 64) before its gradients.  The
 *                  segment length is chosen so that those fit 4 GiB; the
 *                  workspace adds the per-segment states (num_seqs x H x Dk
 *                  x Dv fp32 each) when there is more than one segment.  An
 *                  input that fits one segment runs as one pass.
 *
 * kda_backward_ex / kda_backward_workspace_size_ex take a
 * kda_prefill_options (NULL = automatic): segment_chunks fixes the segment
 * length, segment_bytes the budget of one segment's intermediates;
 * value_block must be 0.  The workspace size depends only on the arguments.
 */
kda_status kda_backward_workspace_size(int B, int T, int H, int Dk, int Dv,
                                       int num_seqs,
                                       const int32_t* cu_seqlens_host,
                                       int chunk_size, size_t* bytes);

kda_status kda_backward(const void* q, const void* k, const void* v,
                        const float* g, const float* beta,
                        const float* initial_state, const float* d_o,
                        const float* d_final_state, float* dq, float* dk,
                        float* dv, float* dg, float* dbeta,
                        float* d_initial_state, const int32_t* cu_seqlens,
                        const int32_t* cu_seqlens_host, int B, int T, int H,
                        int Dk, int Dv, int num_seqs, int chunk_size,
                        kda_dtype in_dtype, void* workspace,
                        size_t workspace_bytes, void* stream /* hipStream_t */);

kda_status kda_backward_workspace_size_ex(int B, int T, int H, int Dk, int Dv,
                                          int num_seqs,
                                          const int32_t* cu_seqlens_host,
                                          int chunk_size,
                                          const kda_prefill_options* options,
                                          size_t* bytes);

kda_status kda_backward_ex(const void* q, const void* k, const void* v,
                           const float* g, const float* beta,
                           const float* initial_state, const float* d_o,
                           const float* d_final_state, float* dq, float* dk,
                           float* dv, float* dg, float* dbeta,
                           float* d_initial_state, const int32_t* cu_seqlens,
                           const int32_t* cu_seqlens_host, int B, int T, int H,
                           int Dk, int Dv, int num_seqs, int chunk_size,
                           kda_dtype in_dtype,
                           const kda_prefill_options* options, void* workspace,
                           size_t workspace_bytes,
                           void* stream /* hipStream_t */);

/*
 * General diagonal-plus-low-rank (DPLR) recurrence, chunked forward pass:
 *
 *     S_t = (Diag(exp g_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t
 *
 * (zeroshot.it.com deep-dive, section 3.2 "DPLR Structure"; greeksharifa
 * summary, section 6.2 "Relation to DPLR").  KDA is the case a = beta k,
 * b = exp(g) k with the write beta k v^T; the general form needs four
 * intra-chunk matrices where KDA needs two.  fp32 arithmetic in per-chunk
 * planes (the same pipeline as kda_prefill_chunk_fp32), exact for any decay
 * strength (chunks whose decay span exceeds 40 evaluate their intra-chunk
 * matrices pair by pair).
 *
 * Arguments as in kda_prefill, plus a, b [B*T, H, Dk] in_dtype; o is float32.
 * The workspace (dplr_prefill_workspace_size) holds fp32 planes of every
 * chunk: about 624 KB per chunk and head at Dk = Dv = 128, C = 64.
 */
kda_status dplr_prefill_workspace_size(int B, int T, int H, int Dk, int Dv,
                                       int num_seqs,
                                       const int32_t* cu_seqlens_host,
                                       int chunk_size, size_t* bytes);

kda_status dplr_prefill(const void* q, const void* k, const void* v,
                        const void* a, const void* b, const float* g, float* o,
                        const float* initial_state, float* final_state,
                        const int32_t* cu_seqlens,
                        const int32_t* cu_seqlens_host, int B, int T, int H,
                        int Dk, int Dv, int num_seqs, int chunk_size,
                        kda_dtype in_dtype, void* workspace,
                        size_t workspace_bytes, void* stream /* hipStream_t */);

/*
 * One general DPLR step for N independent sequences (generation):
 *   S <- Diag(exp g) S - a (b^T S) + k v^T;   o = S^T q
 * q, k, a, b, g [N, H, Dk] (g float32, the others in_dtype); v [N, H, Dv];
 * state [N, H, Dk, Dv] float32, updated in place; o [N, H, Dv] out_dtype.
 * Dk == Dv in {64, 128}.
 */
kda_status dplr_decode_step(const void* q, const void* k, const void* v,
                            const void* a, const void* b, const float* g,
                            float* state, void* o, int N, int H, int Dk, int Dv,
                            kda_dtype in_dtype, kda_dtype out_dtype,
                            void* stream /* hipStream_t */);

/*
 * KDA through the same fp32 chunk pipeline as dplr_prefill, with its tied
 * structure (two intra-chunk matrices): the like-for-like baseline for the
 * general form, and an fp32-arithmetic KDA forward.  Arguments as in
 * kda_prefill (o float32); workspace: dplr_prefill_workspace_size.
 */
kda_status kda_prefill_chunk_fp32(const void* q, const void* k, const void* v,
                                  const float* g, const float* beta, float* o,
                                  const float* initial_state,
                                  float* final_state,
                                  const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_host, int B,
                                  int T, int H, int Dk, int Dv, int num_seqs,
                                  int chunk_size, kda_dtype in_dtype,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream /* hipStream_t */);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
