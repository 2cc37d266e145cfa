/*
 * rda.h -- C ABI of librda.so: the RDA gated-delta token mixer on MI355X.
 *
 * RDA ("Raon Delta Attention") is the linear-attention token mixer of the
 * Raon-1 models.  The "Raon-1 nano" teardown page (ai.satyajit.si), section
 * "The other 1.5B: a hybrid built to forget", orders its recurrent step:
 * scale the matrix state by the decay, take the residual e = v - S'k of the
 * scaled state S' at the key, and add the rank-one update b e k^T (b is the
 * page's beta).  Section "The cache is small if the runtime keeps it small"
 * of the same page fixes the state as 16 heads x 128 x 128 fp32 per layer,
 * carried across calls; the "Raon-1-nano-gguf" page's spec table gives the
 * 16 heads of dimension 128, and its Transformers section notes that the
 * plain PyTorch path walks prompt tokens one at a time.  With a scalar decay
 * a_t and write strength b_t per token and head the step is the gated delta
 * rule
 *
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
 *
 * (read-out after the update; no query scale; q and k are used as given --
 * callers L2-normalise them).  rda_prefill evaluates it for whole prompts in
 * chunks of 64 tokens (WY / UT-transform form on bf16 MFMA); rda_decode_step
 * applies one token in place (both also with a per-channel decay:
 * rda_prefill_diag, rda_decode_step_diag); rda_decode_tokens applies a few (a verify of
 * drafted tokens) in one pass over the state (rda_decode_tokens_diag with the
 * per-channel decay); rda_prologue produces their
 * inputs from the raw projections (short convolution, q/k norm, gates), and
 * rda_output_norm_gate is the block's output norm and gate on the mixer's
 * output.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers to contiguous row-major memory,
 *   16-byte aligned.  The caller owns every buffer; the library allocates no
 *   device memory (rda_prefill takes a caller-provided workspace).
 * - Layouts: tokens q, k [T, H, dk], v [T, H, dv]; gates a, b [T, H] fp32;
 *   states [N, H, dv, dk] fp32 with S[i][j], i = value channel (row),
 *   j = key channel (column); outputs o [T, H, dv] fp32.
 * - Only dk = dv = 128 is supported (RDA_ERR_UNSUPPORTED otherwise).
 * - Work is enqueued asynchronously on `stream` (0 = the null stream); no
 *   entry point synchronises the host.  Entry points only launch kernels (no
 *   allocation, memset or copy), so a caller may capture them in a HIP
 *   graph and replay it.  Argument checks run on the host
 *   before anything is enqueued; on an error nothing is launched.  Launch
 *   failures return RDA_ERR_HIP.  Nothing aborts, throws or prints.
 * - Gates must satisfy a in (0, 1] and b in [0, 1]; other values are not
 *   checked and give unspecified (but memory-safe) results.
 * - Entry points hold no mutable global state and are thread-safe.
 */
#ifndef RDA_H
#define RDA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RDA_ABI_VERSION 1
#define RDA_CHUNK 64      /* tokens per prefill chunk */
#define RDA_HEAD_DIM 128  /* the only supported dk = dv */
#define RDA_DECODE_MAX_TOKENS 64  /* tokens per rda_decode_tokens call (one chunk) */
#define RDA_CONV_MAX_WIDTH 4      /* taps of the prologue's short convolution */

typedef enum {
    RDA_OK = 0,
    RDA_ERR_NULL = 1,        /* a required pointer is NULL */
    RDA_ERR_SHAPE = 2,       /* a size is negative / zero where not allowed / overflows */
    RDA_ERR_UNSUPPORTED = 3, /* a valid shape this build does not implement (dk, dv != 128) */
    RDA_ERR_DTYPE = 4,       /* unknown rda_dtype */
    RDA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than rda_prefill_workspace_bytes */
    RDA_ERR_ALIGN = 6,       /* a pointer is not 16-byte aligned */
    RDA_ERR_HIP = 7,         /* a HIP launch reported an error */
    RDA_ERR_ALIAS = 8,       /* outputs overlap inputs (other than S_final == S0) */
    RDA_ERR_VALUE = 9,       /* a scalar argument out of range (eps, gate activation) */
    RDA_ERR_TOO_LARGE = 10   /* sizes need more than rda_prefill_noalloc's fixed scratch */
} rda_status;

typedef enum { RDA_BF16 = 0, RDA_FP32 = 1 } rda_dtype;

/* Stages of one rda_prefill call, in launch order (for rda_prefill_profiled). */
typedef enum {
    RDA_STAGE_TABLE = 0, /* chunk table from cu_seqlens (empty for one bf16 sequence
                            with cu_seqlens NULL: the prep kernel writes the table) */
    RDA_STAGE_PREP = 1,  /* per-chunk intra-chunk solve and WY products (parallel) */
    RDA_STAGE_WALK = 2,  /* inter-chunk state passing and outputs (sequential per sequence) */
    RDA_NUM_STAGES = 3
} rda_stage;

/* RDA_ABI_VERSION of the loaded library. */
int rda_abi_version(void);

/* Static English text for a status code (never NULL). */
const char* rda_status_string(int status);

/* Upper bound on the number of 64-token chunks of a packed batch:
 * floor((total_tokens + 63 * num_seqs) / 64).  Returns -1 on bad sizes. */
int32_t rda_max_chunks(int32_t num_seqs, int32_t total_tokens);

/* Workspace bytes rda_prefill needs for these sizes (0 on bad sizes).  The
 * workspace holds the chunk table and the per-chunk WY factors; its contents
 * need no initialisation and are garbage after the call. */
size_t rda_prefill_workspace_bytes(int32_t num_seqs, int32_t total_tokens,
                                   int32_t num_heads, int32_t dk, int32_t dv);

/*
 * Chunked prefill over a packed batch of variable-length sequences.
 *
 * The "Raon-1-nano-gguf" model card (Transformers section) notes that the
 * plain PyTorch path processes a prompt one token at a time, which makes
 * long prompts slow; this entry point computes the same recurrence (the
 * step ordered as in the teardown's section "The other 1.5B: a hybrid built
 * to forget") for every token of a prompt in one call, with the chunks of 64
 * tokens handled in parallel where the algebra allows and only the state
 * passed from chunk to chunk in sequence.
 *
 *   q, k        [total_tokens, H, dk], v [total_tokens, H, dv], dtype qkv_dtype
 *               (RDA_BF16 or RDA_FP32; fp32 values are fed to MFMA as exact
 *               bf16 hi + lo pairs)
 *   a, b        [total_tokens, H] fp32 gates
 *   cu_seqlens  device int32 [num_seqs + 1] token offsets, or NULL for one
 *               sequence of total_tokens (then num_seqs must be 1).  Contents
 *               are trusted (cu[0] = 0, non-decreasing, cu[N] = total_tokens;
 *               the Python binding checks this on a host copy) but never read
 *               or used out of bounds.  Zero-length sequences are allowed and
 *               return S_final = S0.
 *   S0          [num_seqs, H, dv, dk] fp32 initial states, or NULL for zeros
 *   o           [total_tokens, H, dv] fp32 output
 *   S_final     [num_seqs, H, dv, dk] fp32 output, or NULL to skip; may be the
 *               same pointer as S0 (in-place resume), no other overlap allowed
 *   workspace   device scratch of at least rda_prefill_workspace_bytes(...)
 * total_tokens = 0 is allowed (only S_final is written).
 *
 * The state passing between chunks is sequential per (sequence, head) and
 * gives each pair 8 workgroups.  One bf16 sequence without offsets with few
 * heads (H <= 4 with at least 16 chunks per segment; the plan is fixed by
 * total_tokens and H) is instead cut into P = 4..16 segments. Each segment is
 * walked from zero and, with its values taken as zero, from the identity;
 * the segments' affine maps are chained, and each segment is walked again from
 * its true starting state for the outputs. This is the segment-summary form
 * in the state-passing row of the chunked method (one long prompt's share of
 * heads on one GPU). It gives the same result up to rounding, and
 * rda_prefill_workspace_bytes(1, T, H) includes its three [P, H, dv, dk]
 * state arrays.  With more heads (at least 32 chunks and at least 64 CUs
 * left idle by the walk's 8 H workgroups) the same input instead runs the
 * prep of the first chunks, then their walk beside the prep of the rest on
 * the idle CUs, then the walk of the rest; the result is bitwise that of the
 * one-pass walk, and the workspace includes one [H, dv, dk] state.  Passing
 * cu_seqlens = {0, T} keeps the one-pass walk.
 */
rda_status rda_prefill(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                       const float* a, const float* b,
                       const int32_t* cu_seqlens, int32_t num_seqs,
                       int32_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                       const float* S0, float* o, float* S_final,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * rda_prefill with per-stage timing events: when `stage_events` is non-NULL
 * it points to 2 * RDA_NUM_STAGES events; stage s records stage_events[2s]
 * before its first kernel and stage_events[2s+1] after its last, on
 * `stream` (NULL entries are skipped).  The kernels are those rda_prefill
 * runs: in the plan that preps later chunks beside the walk, the table
 * stage is empty, the prep stage is the prep of the first chunks and the
 * walk stage spans the walk launches.  Results are identical to
 * rda_prefill.
 */
rda_status rda_prefill_profiled(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                                const float* a, const float* b,
                                const int32_t* cu_seqlens, int32_t num_seqs,
                                int32_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                                const float* S0, float* o, float* S_final,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t const* stage_events);

/*
 * rda_prefill for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as rda_prefill, without the workspace:
 * the chunk table and the per-chunk factors go to a fixed device array of
 * RDA_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, allocated when
 * the library's code is loaded on that GPU and held until the process
 * ends).  The call itself allocates nothing (no hipMalloc / hipFree, no
 * allocating library routine).  Sizes whose rda_prefill_workspace_bytes
 * exceed RDA_NOALLOC_SCRATCH_BYTES return RDA_ERR_TOO_LARGE before anything
 * is enqueued (for one sequence of 16 heads that is a prompt of up to about
 * 7800 tokens).
 * The first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress) and keeps its address; a failed lookup returns
 * RDA_ERR_HIP.  Every call on one GPU uses the same array: calls that may
 * overlap in time on one GPU (different streams, or threads without
 * ordering) race on it and give undefined results, so serialise them on
 * one stream.  The array needs no clearing between calls (every byte a call
 * reads is written earlier in the same call).
 */
#define RDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
rda_status rda_prefill_noalloc(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                               const float* a, const float* b,
                               const int32_t* cu_seqlens, int32_t num_seqs,
                               int32_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                               const float* S0, float* o, float* S_final, hipStream_t stream);

/*
 * One decode step: the recurrence for a single token per (batch, head),
 * updating the state in place in one read-modify-write pass over it.  The
 * teardown's section "The cache is small if the runtime keeps it small"
 * describes the generation-time cost this serves: per RDA layer the runtime
 * carries the 16 x 128 x 128 fp32 state from token to token (1 MiB per
 * sequence), so each generated token reads and rewrites it once.
 *
 *   q, k [batch, H, dk], v [batch, H, dv] (qkv_dtype); a, b [batch, H] fp32
 *   S    [batch, H, dv, dk] fp32, read and overwritten with the new state
 *   o    [batch, H, dv] fp32 output (o = S_new q)
 * batch = 0 is allowed (nothing is launched); batch x H above 2^30 - 1 is
 * rejected with RDA_ERR_SHAPE.
 */
rda_status rda_decode_step(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                           const float* a, const float* b,
                           int32_t batch, int32_t num_heads, int32_t dk, int32_t dv,
                           float* S, float* o, hipStream_t stream);

/*
 * Several tokens per sequence in one pass over the state: the decode step
 * for a verify of drafted tokens.  The "Raon-1-nano-gguf" model card's
 * llama.cpp section runs the model with multi-token prediction proposing
 * two drafts per step, and the Raon-1-mini vLLM support article discusses
 * the speculative-decoding draft model; verifying such a step feeds the
 * current token plus its drafts (tokens = 1 + drafts) through the mixer
 * and keeps the state only up to the last accepted token.  The recurrence
 * is the one above, applied token after token; each state is read once and
 * written at most once.
 *
 *   q, k [batch, tokens, H, dk], v [batch, tokens, H, dv] (qkv_dtype);
 *   a, b [batch, tokens, H] fp32 -- the packed layout of `batch` sequences
 *        of `tokens` tokens each
 *   S_in   [batch, H, dv, dk] fp32 state before the first token (read)
 *   accept device int32 [batch] or NULL: tokens to commit per sequence,
 *          clamped to [0, tokens]; NULL commits all `tokens`
 *   S_out  [batch, H, dv, dk] fp32 or NULL: receives the state after the
 *          first accept[n] tokens of sequence n.  S_out == S_in updates in
 *          place; NULL leaves every state untouched (read-only verify)
 *   o      [batch, tokens, H, dv] fp32 or NULL: o_t = S_t q_t for every
 *          token, accepted or not.  NULL skips the outputs (q is then not
 *          read and may be NULL): a commit after a read-only verify
 * A verify whose accept counts are only known from its outputs runs as two
 * calls: S_out = NULL with o, then accept with S_out and o = NULL.
 * tokens in [0, RDA_DECODE_MAX_TOKENS] (longer runs belong to rda_prefill);
 * tokens = 1 with S_out == S_in and accept = NULL is rda_decode_step.
 * S_in may be NULL only when batch = 0; S_out and o may not both be NULL.
 * S_out and S_in must be the same pointer or disjoint (RDA_ERR_ALIAS).
 */
rda_status rda_decode_tokens(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                             const float* a, const float* b, int32_t batch, int32_t tokens,
                             int32_t num_heads, int32_t dk, int32_t dv, const float* S_in,
                             float* S_out, const int32_t* accept, float* o, hipStream_t stream);

/*
 * Per-channel (diagonal) decay: the variants of rda_prefill and
 * rda_decode_step whose decay is a vector over the key channels,
 * alpha_t in (0, 1]^dk, instead of one scalar per token and head.  The
 * Raon-1 mini vLLM article calls RDA a modification of Kimi Delta Attention,
 * whose decay is per channel, and the tiny-model card prints a low-rank
 * decay projection whose output has the heads' key width.  The step, in the
 * teardown's order:
 *
 *     S' = S_{t-1} diag(alpha_t),  e = v_t - S' k_t,  S_t = S' + b_t e k_t^T,
 *     o_t = S_t q_t
 *
 * Arguments as in rda_prefill / rda_decode_step, with alpha [total_tokens, H,
 * dk] (prefill) or [batch, H, dk] (decode) fp32 in place of a, q, k, v in
 * bf16 or fp32 (fp32 values keep their full precision through the chunked
 * products), and the prefill's own workspace size.  Any alpha in (0, 1] is
 * safe: the chunked prefill never
 * forms a decay factor above e^60 (it falls back to exact per-element
 * factors where a 16-token block decays by more than that).  One sequence
 * without offsets with few heads takes the segmented state pass described
 * at rda_prefill (same plan; its workspace size includes the state arrays);
 * with more heads, the overlapped plan described there, in growing chunk
 * ranges: the prep of the first range, then one walk launch per range beside
 * the prep of the next on the idle CUs (bitwise the one-pass result; the
 * workspace includes one [H, dv, dk] state).
 */
size_t rda_prefill_diag_workspace_bytes(int32_t num_seqs, int32_t total_tokens,
                                        int32_t num_heads, int32_t dk, int32_t dv);
rda_status rda_prefill_diag(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                            const float* alpha, const float* b, const int32_t* cu_seqlens,
                            int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                            int32_t dk, int32_t dv, const float* S0, float* o, float* S_final,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
rda_status rda_decode_step_diag(const void* q, const void* k, const void* v,
                                rda_dtype qkv_dtype, const float* alpha, const float* b,
                                int32_t batch, int32_t num_heads, int32_t dk, int32_t dv,
                                float* S, float* o, hipStream_t stream);
/*
 * rda_decode_tokens with the per-channel decay: alpha [batch, tokens, H, dk]
 * fp32 in place of a (token t of sequence n, head h at row
 * (n * tokens + t) * H + h), every other argument, layout, accept rule and
 * error as in rda_decode_tokens.  Its result equals rda_prefill_diag over the
 * same tokens taken as batch sequences of `tokens` tokens each.
 */
rda_status rda_decode_tokens_diag(const void* q, const void* k, const void* v,
                                  rda_dtype qkv_dtype, const float* alpha, const float* b,
                                  int32_t batch, int32_t tokens, int32_t num_heads, int32_t dk,
                                  int32_t dv, const float* S_in, float* S_out,
                                  const int32_t* accept, float* o, hipStream_t stream);

/* Activation after the prologue's short convolution. */
typedef enum {
    RDA_CONV_ACT_NONE = 0,
    RDA_CONV_ACT_SILU = 1  /* y * sigmoid(y) */
} rda_conv_act;

/*
 * The prologue of the RDA block: the steps between its projections and the
 * recurrence, producing the inputs of rda_prefill / the decode entry points.
 * The Raon-1 nano teardown keeps a short convolution window per layer beside
 * the recurrent state (section "The cache is small if the runtime keeps it
 * small") and gives the decoupled gates -- erase strength b =
 * sigmoid(beta_raw), a write gate sigmoid(beta_raw + delta) / sigmoid(beta_raw)
 * scaling the value -- and the decay bounded below by -5 in log space
 * (section "The other 1.5B: a hybrid built to forget"); the Raon-1 mini vLLM
 * article applies the write gate after the convolution, so the history holds
 * raw tokens, and keeps that history in bf16.  Per token t of sequence n,
 * tensor x in (q, k, v), head h, channel c:
 *
 *   y   = sum_{i<K} w[x][h][c][i] * raw_x[t - (K-1) + i]   (raw tokens before
 *         the sequence's first token come from its history)
 *   y   = silu(y) with RDA_CONV_ACT_SILU
 *   q,k = y / sqrt(sum_c y^2 + l2_eps);   v = y * sig(beta_raw + delta) / sig(beta_raw)
 *   b   = sig(beta_raw);   a = exp(max(g_log, decay_floor))
 *
 *   x_q, x_k, x_v  raw projections [total_tokens, H, d] bf16 (x_dtype must be
 *                  RDA_BF16)
 *   conv_w         [3, H, d, K] fp32: the q, k and v depthwise weights, tap
 *                  K-1 multiplying the current token; K = conv_width in
 *                  1..RDA_CONV_MAX_WIDTH
 *   hist_in        [num_seqs, 3, K-1, H, d] bf16: the K-1 raw tokens before
 *                  each sequence, oldest first (q, k, v), or NULL for zeros
 *   hist_out       same shape, or NULL to skip: the raw tokens at each
 *                  sequence's last K-1 positions (the newest of hist_in where
 *                  a sequence is shorter; hist_in itself for an empty one).
 *                  It may be hist_in itself only when every sequence has one
 *                  token (cu_seqlens NULL and total_tokens = num_seqs);
 *                  otherwise any overlap is RDA_ERR_ALIAS
 *   beta_raw, g_log  [total_tokens, H] fp32; delta [total_tokens, H] fp32 or
 *                  NULL (write gate 1)
 *   decay_floor    log-space floor of the decay (-5 per the teardown; -INF
 *                  for none; NaN is RDA_ERR_VALUE); l2_eps >= 0 and finite
 *   cu_seqlens     device int32 [num_seqs + 1] offsets (trusted as in
 *                  rda_prefill, never read or used out of bounds), or NULL
 *                  for num_seqs sequences of total_tokens / num_seqs tokens
 *                  each (the layouts of rda_decode_step, one token, and
 *                  rda_decode_tokens); total_tokens must then divide evenly
 *   q, k, v        outputs [total_tokens, H, d] bf16 (round to nearest even),
 *                  the inputs of rda_prefill / rda_decode_*; a, b outputs
 *                  [total_tokens, H] fp32
 * d must be 128.  total_tokens = 0 is allowed (only hist_out is written).
 */
rda_status rda_prologue(const void* x_q, const void* x_k, const void* x_v, rda_dtype x_dtype,
                        const float* conv_w, int32_t conv_width, int32_t conv_act,
                        const void* hist_in, void* hist_out, const float* beta_raw,
                        const float* delta, const float* g_log, float decay_floor, float l2_eps,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                        int32_t num_heads, int32_t d, void* q, void* k, void* v, float* a,
                        float* b, hipStream_t stream);

/*
 * One decode step with the prologue in front: rda_prologue for one token
 * per sequence (the decode layout, cu_seqlens NULL, total_tokens = batch)
 * followed by rda_decode_step, in one launch and one pass over the state,
 * without q, k, v, a, b reaching memory.  The teardown's section "The cache
 * is small if the runtime keeps it small" counts the short convolution
 * windows beside the recurrent state as the per-sequence decode cache; this
 * entry point carries both, the state S and the history, in and out.
 *
 *   x_q, x_k, x_v  raw projections [batch, H, d] bf16 (x_dtype must be RDA_BF16)
 *   conv_w, conv_width, conv_act, beta_raw, delta, g_log, decay_floor, l2_eps
 *                  as in rda_prologue ([batch, H] for the gates)
 *   hist_in        [batch, 3, K-1, H, d] bf16 or NULL (zeros)
 *   hist_out       same shape or NULL (not kept); may be hist_in itself (the
 *                  history moves on by one token in place); any other overlap
 *                  with an argument is RDA_ERR_ALIAS
 *   S              [batch, H, d, d] fp32, updated in place
 *   o              [batch, H, d] fp32
 * The result equals rda_prologue followed by rda_decode_step on its outputs
 * bit for bit (the same arithmetic, and q, k, v rounded to bf16 as the
 * prologue writes them).  batch = 0 is allowed; d must be 128.
 */
rda_status rda_decode_step_prologue(const void* x_q, const void* x_k, const void* x_v,
                                   rda_dtype x_dtype, const float* conv_w, int32_t conv_width,
                                   int32_t conv_act, const void* hist_in, void* hist_out,
                                   const float* beta_raw, const float* delta, const float* g_log,
                                   float decay_floor, float l2_eps, int32_t batch,
                                   int32_t num_heads, int32_t dk, int32_t dv, float* S, float* o,
                                   hipStream_t stream);

/* Activation of the output gate in rda_output_norm_gate. */
typedef enum {
    RDA_GATE_SIGMOID = 0,  /* sigmoid(g) */
    RDA_GATE_SILU = 1,     /* g * sigmoid(g) */
    RDA_GATE_NONE = 2      /* no gate: the RMS norm alone */
} rda_gate_act;

/*
 * The output epilogue of the RDA block, applied to the mixer's output rows:
 * per row of one head (dv channels) an RMS normalisation with epsilon and a
 * per-channel weight, times an activation of the output gate.  The
 * tiny-random/raon-1-mini model card, section "Printing the model", lists
 * the block's o_norm (an RMS norm over the head dimension, eps 1e-5, with a
 * weight of the head dimension's size) and the g_proj projection producing
 * the gate; the card does not print the gate's activation, hence `act`.
 *
 *     out_c = o_c / sqrt(mean_c'(o_c'^2) + eps) * weight_c * act(g_c)
 *
 *   o       [rows, dv] fp32: the mixer's output, rows = tokens x heads
 *           (rda_prefill's o) or batch x heads (the decode entry points')
 *   g       [rows, dv] in g_dtype (bf16 or fp32); may be NULL with
 *           RDA_GATE_NONE (then g_dtype is ignored)
 *   weight  [dv] fp32, shared by the heads; NULL means 1
 *   eps     finite and >= 0 (RDA_ERR_VALUE otherwise); act an rda_gate_act
 *   out     [rows, dv] in out_dtype (bf16, rounded to nearest even, or fp32).
 *           An fp32 out may be o itself (in place); any other overlap with
 *           an input is RDA_ERR_ALIAS.
 * rows = 0 is allowed (nothing is launched); dv must be 128.
 */
rda_status rda_output_norm_gate(const float* o, const void* g, rda_dtype g_dtype,
                                const float* weight, float eps, int32_t act, int64_t rows,
                                int32_t dv, void* out, rda_dtype out_dtype, hipStream_t stream);

/* Workspace bytes rda_prefill_norm_gate needs (0 on bad sizes): that of
 * rda_prefill plus 2 bytes per output element for the 16-bit form below. */
size_t rda_prefill_norm_gate_workspace_bytes(int32_t num_seqs, int32_t total_tokens,
                                             int32_t num_heads, int32_t dk, int32_t dv);

/*
 * rda_prefill followed by rda_output_norm_gate on its output, without the
 * fp32 output: the block's mixer and its o_norm / gate (the
 * tiny-random/raon-1-mini model card, section "Printing the model") in one
 * call.  The walk stores each token-head row in 16 bits per channel, in the
 * workspace: each 16-channel slice scaled by a power of two that puts its
 * largest magnitude in [0.5, 1), as fp16, with the scale's exponent carried
 * in the lowest bit of the slice's first 8 values.  A pass over that form
 * restores the values, takes the RMS norm and applies the weight and the
 * gate; for one bf16 sequence whose walk leaves CUs idle, most of that pass
 * runs beside the walk over the rows already walked.
 *
 *   q, k, v, a, b, cu_seqlens, num_seqs, total_tokens, num_heads, dk, dv,
 *   S0, S_final   as for rda_prefill
 *   g, g_dtype, weight, eps, act, out, out_dtype
 *                 as for rda_output_norm_gate with rows = total_tokens x
 *                 num_heads; out [total_tokens, H, dv] may not overlap any
 *                 other argument or the workspace
 *   workspace     at least rda_prefill_norm_gate_workspace_bytes(...)
 * Errors: those of both entry points, checked before anything is enqueued.
 * The result differs from the two calls' by the 16-bit form: at most 2^-11
 * relative per value from the fp16 rounding, plus 2^-10 on the 8 values of a
 * slice that carry its exponent, below the output's bf16 rounding.  A slice
 * whose largest magnitude is an fp32 subnormal counts as zeros.
 */
rda_status rda_prefill_norm_gate(const void* q, const void* k, const void* v, rda_dtype qkv_dtype,
                                 const float* a, const float* b,
                                 const int32_t* cu_seqlens, int32_t num_seqs,
                                 int32_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                                 const float* S0, const void* g, rda_dtype g_dtype,
                                 const float* weight, float eps, int32_t act, void* out,
                                 rda_dtype out_dtype, float* S_final, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * Test hook: the chunk table rda_prefill builds from cu_seqlens.
 *   out               device int32 [rda_max_chunks(...), 4]; row c =
 *                     (sequence, first token, valid length 1..64, chunk index
 *                     within its sequence) for c < *num_chunks, (-1, 0, 0, 0) after
 *   out_seq_offsets   device int32 [num_seqs + 1]: first chunk of each sequence
 *                     (exclusive prefix sum of ceil(len / 64)); required
 *   out_num_chunks    device int32 [1]: number of chunks
 * cu_seqlens may be NULL (one sequence of total_tokens, num_seqs = 1).
 */
rda_status rda_chunk_table(const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                           int32_t* out, int32_t* out_seq_offsets, int32_t* out_num_chunks,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RDA_H */
