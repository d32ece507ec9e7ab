/*
 * spec.h -- C ABI of the MI355X (gfx950) speculative-decoding verify step.
 *
 * The calls follow the statement of the problem on the pages:
 *   - a drafter proposes K tokens one at a time ("Speculative Decoding on Apple Silicon:
 *     119% Faster on Qwen3.8, Until It Isn't", section "How speculative decoding works");
 *   - the target scores all of them in one batched pass, the same way it reads a prompt
 *     ("What is Speculative Decoding and How Does a Draft Model Work?", section "#2");
 *   - the longest agreeing prefix is kept plus one token of the target's own: greedy
 *     match at temperature 0 (same page, "#3"), or acceptance with probability
 *     min(1, p/q) and a replacement drawn from the clipped, rescaled difference of the
 *     two distributions ("Qwen3.5 and Qwen3.6 MTP head reaches 1.4x on Apple Silicon after
 *     three fixes", section "The verify was wrong under sampling"), with the same
 *     temperature / top_k / top_p truncation on both sides (same page, "Truncation has to
 *     match on both sides");
 *   - the key/value cache is rolled back by slicing the rejected entries off its end
 *     ("Speculative Decoding on Apple Silicon: 119% Faster...", section "Why this needed a
 *     patch to mlx_lm at all").
 *
 * Conventions for every call:
 *   - "device" pointers are GPU (HBM) addresses, "host" pointers are CPU addresses.
 *   - Every device buffer is owned by the caller, who keeps it alive until the work that
 *     uses it has finished on the stream.  The library never allocates device memory: a
 *     context lives in a caller-provided workspace, and model weights are borrowed, never
 *     copied ("Qwen3.5 and Qwen3.6 MTP head...", section "Duplicate weights in unified
 *     memory": drafting must reuse the already-loaded weights).
 *   - Work is enqueued on the stream given at spec_init (or per call for the stateless
 *     entry points) and the call returns at once; outputs are valid once that stream has
 *     been synchronized.  Only the calls documented as synchronizing wait on the stream.
 *   - Matrices are row-major, weights in the [out_features, in_features] layout.
 *   - Return value: SPEC_OK (0) or a negative SPEC_E_* code.  Arguments are validated on
 *     the host before anything is enqueued; on an error nothing is enqueued and the
 *     context (if any) keeps a message readable with spec_last_error.  No C++ exception
 *     crosses this interface.  One context per stream; calls on one context are not
 *     thread-safe.
 */
#ifndef SPEC_H_
#define SPEC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------------------ */
#define SPEC_OK 0
#define SPEC_E_INVAL (-1)       /* bad argument (null pointer, bad shape, bad sampler)   */
#define SPEC_E_RANGE (-2)       /* would overflow the cache, trim past the end, too big  */
#define SPEC_E_UNSUPPORTED (-3) /* valid request outside what the kernels implement      */
#define SPEC_E_STATE (-4)       /* call out of order (e.g. accept before verify)         */
#define SPEC_E_HIP (-5)         /* a HIP runtime call failed                             */

/* ---- enums ---------------------------------------------------------------------------- */
#define SPEC_DTYPE_F32 0  /* weights, cache and GEMM inputs in float32                    */
#define SPEC_DTYPE_BF16 1 /* bf16 weights and cache, bf16 GEMM inputs, fp32 accumulation  */

/* Storage of the projection and LM-head weights (spec_model_desc.weights).  The pages' runs
 * decode with quantized weights ("Speculative Decoding on Apple Silicon", section
 * "Reproducing this"; "What is Speculative Decoding and How Does a Draft Model Work?", section
 * "The demo, draft model on and off with two pairings"):
 * a verify then reads fewer weight bytes per cycle.  The byte format here is the E4M3 type
 * of the OCP 8-bit floating point specification, which gfx950 converts in hardware.  FP8_ROW
 * models run the SPEC_SCHED_STREAM projections whatever the schedule; they need reduction
 * lengths of 2048 or 4096 for the normalized projections (QKV, gate/up, LM head) and whole
 * 2 KB stages for the rest, at most 16 rows per forward, and a drafter other than
 * SPEC_DRAFT_MTP; else spec_init returns SPEC_E_UNSUPPORTED. */
#define SPEC_WEIGHTS_NATIVE 0 /* in the model's dtype                                      */
#define SPEC_WEIGHTS_FP8_ROW 1 /* bf16 models only: one byte per weight, an OCP FP8 E4M3
                                  code (1 sign, 4 exponent bits of bias 7, 3 mantissa bits;
                                  no infinities, S.1111.111 is NaN), and one float32 scale
                                  per output row: weight[r][k] = decode(code[r][k]) * scale[r].
                                  The embedding and the norm gains stay bf16; the LM head
                                  must be its own tensor (not tied to the embedding). */

#define SPEC_DRAFT_NONE 0  /* no drafter: verify_step at k = 0 is plain decoding          */
#define SPEC_DRAFT_MODEL 1 /* a separate, smaller decoder with the same vocabulary         */
#define SPEC_DRAFT_MTP 2   /* the target's own multi-token-prediction layer               */
#define SPEC_DRAFT_NGRAM 3 /* n-gram lookup in the context                                */

#define SPEC_TOPK_MAX 64   /* largest top_k the truncation kernels keep                   */
#define SPEC_MAX_K 16      /* largest number of drafts per cycle                          */

/* near-tie / status flag bits written per row or per sequence */
#define SPEC_FLAG_ACCEPT_TIE 1u  /* |u - p/q| < 1e-6 at an accept test                  */
#define SPEC_FLAG_SAMPLE_TIE 2u  /* |running sum - u*Z| < 1e-6 at the deciding CDF step */
#define SPEC_FLAG_TOPP_TIE 4u    /* |exclusive running sum - top_p| < 1e-6 at the cut   */
#define SPEC_FLAG_BAD_ROW 8u     /* row had NaN / +inf, or no finite logit              */

/* ---- model description (all weight pointers are device, borrowed) ------------------- */
typedef struct spec_layer_weights {
  const void* attn_norm; /* [d_model]                      */
  const void* wq;        /* [n_q_heads*head_dim, d_model]  */
  const void* wk;        /* [n_kv_heads*head_dim, d_model] */
  const void* wv;        /* [n_kv_heads*head_dim, d_model] */
  const void* wo;        /* [d_model, n_q_heads*head_dim]  */
  const void* ffn_norm;  /* [d_model]                      */
  const void* wg;        /* [d_ffn, d_model]               */
  const void* wu;        /* [d_ffn, d_model]               */
  const void* wd;        /* [d_model, d_ffn]               */
} spec_layer_weights;

/* Row scales of one layer's projections for SPEC_WEIGHTS_FP8_ROW (device float32 arrays,
 * borrowed): one entry per output row of the matrix of the same name. */
typedef struct spec_layer_scales {
  const float* wq; /* [n_q_heads*head_dim]  */
  const float* wk; /* [n_kv_heads*head_dim] */
  const float* wv; /* [n_kv_heads*head_dim] */
  const float* wo; /* [d_model]             */
  const float* wg; /* [d_ffn]               */
  const float* wu; /* [d_ffn]               */
  const float* wd; /* [d_model]             */
} spec_layer_scales;

typedef struct spec_model_desc {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab;
  int32_t dtype;                    /* SPEC_DTYPE_*; every tensor of the model has it     */
  float rms_eps;                    /* RMSNorm epsilon (1e-6 for the Qwen-shaped models)   */
  float rope_theta;                 /* rotate-half RoPE base (1e6)                         */
  const void* embed;                /* [vocab, d_model]                                    */
  const void* lm_head;              /* [vocab, d_model]; may be the embed pointer (tied)   */
  const void* final_norm;           /* [d_model]                                           */
  const spec_layer_weights* layers; /* host array [n_layers]; copied by spec_init          */
  int32_t weights;                  /* SPEC_WEIGHTS_*; zero-initialised descs are native   */
  const float* lm_head_scale;       /* FP8_ROW: [vocab] row scales of lm_head              */
  const spec_layer_scales* layer_scales; /* FP8_ROW: host array [n_layers]; copied      */
} spec_model_desc;

/* Multi-token-prediction layer: concat(RMSNorm(h_t), RMSNorm(E[x_{t+1}])) -> w_proj ->
 * one decoder layer -> RMSNorm -> the target's LM head.  Shares the target's embed and
 * lm_head; d_model and heads are the target's. */
typedef struct spec_mtp_desc {
  const void* norm_h;       /* [d_model]                */
  const void* norm_e;       /* [d_model]                */
  const void* w_proj;       /* [d_model, 2*d_model]     */
  const void* final_norm;   /* [d_model]                */
  spec_layer_weights layer; /* one decoder layer        */
} spec_mtp_desc;

/* temperature <= 0 selects greedy decoding (argmax, lowest id on ties); otherwise the
 * row is divided by temperature, cut to the top_k largest (1..SPEC_TOPK_MAX), softmaxed,
 * cut where the exclusive running sum reaches top_p (0 < top_p <= 1), renormalized. */
typedef struct spec_sampler {
  float temperature;
  int32_t top_k;
  float top_p;
} spec_sampler;

typedef struct spec_ngram_cfg {
  int32_t n_min;     /* shortest match that triggers a draft (3)        */
  int32_t max_match; /* longest match length considered (16)            */
} spec_ngram_cfg;

typedef struct spec_config {
  spec_model_desc target;
  int32_t draft_kind;     /* SPEC_DRAFT_*                                   */
  spec_model_desc draft;  /* used when draft_kind == SPEC_DRAFT_MODEL       */
  spec_mtp_desc mtp;      /* used when draft_kind == SPEC_DRAFT_MTP         */
  spec_ngram_cfg ngram;   /* used when draft_kind == SPEC_DRAFT_NGRAM       */
  spec_sampler sampler;
  uint64_t seed;          /* Philox4x32-10 key for every uniform the method draws */
  int32_t max_batch;      /* sequences per call (B)                         */
  int32_t max_ctx;        /* longest context, in tokens, before a verify    */
  int32_t max_k;          /* largest k passed to draft_step / verify_step   */
} spec_config;

/* A batch of truncated distributions, one row each: row r holds count[r] (id, prob) pairs,
 * ids ascending, at ids[r*cap .. r*cap+count[r]).  Device buffers owned by the caller. */
typedef struct spec_probs {
  int32_t* ids;   /* device [rows * cap] */
  float* probs;   /* device [rows * cap] */
  int32_t* count; /* device [rows]       */
  int32_t cap;    /* row stride; >= top_k (>= 1 for greedy) */
} spec_probs;

typedef struct spec_stats {
  int64_t cycles;           /* accept calls                                   */
  int64_t drafts_attempted; /* sum of k over accept calls and sequences        */
  int64_t drafts_accepted;  /* sum of n                                        */
  int64_t emitted;          /* sum of n + 1                                    */
  int64_t sync_timeouts;    /* non-zero once a grid barrier of the one-launch forward timed
                             * out (its results, and every later one, are invalid); the
                             * calls that synchronize (spec_get_stats, spec_get_lengths, a
                             * draft_step / verify_step that reads the lengths) then return
                             * SPEC_E_HIP, and so does every later draft_step, verify_step,
                             * accept and kv_trim of the context */
} spec_stats;

typedef struct spec_ctx spec_ctx;

/* ---- lifecycle --------------------------------------------------------------------- */

/* Bytes of device workspace spec_init needs for cfg: caches for max_ctx + max_k + 2
 * positions per sequence, activations for max_batch*(max_k+1) rows, partial results of
 * the split attention and of the truncation, lengths and counters.  Host only. */
int spec_workspace_size(const spec_config* cfg /*host*/, size_t* bytes /*host out*/);

/* Validates cfg (head_dim <= 128 and even, d_model and every projection width a multiple
 * of 16 and of 8 elements, n_q_heads a multiple of n_kv_heads, 1 <= max_k <= SPEC_MAX_K,
 * vocab >= top_k, draft vocab == target vocab), copies the weight pointer tables, carves
 * `workspace` (device, >= spec_workspace_size bytes, 256-byte aligned, owned by the
 * caller) and enqueues its zeroing on `stream` (a hipStream_t, NULL = default stream).
 * Sequence lengths start at 0.  *out receives a host-allocated context. */
int spec_init(const spec_config* cfg /*host*/, void* workspace /*device*/, size_t ws_bytes,
              void* stream, spec_ctx** out /*host out*/);

/* Frees the host context (not the workspace, not the weights).  NULL is accepted. */
int spec_destroy(spec_ctx* ctx);

/* Last error message of ctx (NULL ctx: the last spec_init error).  Never NULL. */
const char* spec_last_error(const spec_ctx* ctx);

/* ---- state set-up ------------------------------------------------------------------ */

/* Copies a cache prefix for sequence `seq` of the target (which = 0), the draft model
 * (1) or the MTP layer (2): k, v are device [n_layers, n_kv_heads, length, head_dim] in
 * the model dtype (n_layers = 1 for the MTP layer), keys already rotated.  Sets that
 * cache's length to `length`.  For which = 0 it also sets the sequence's context length;
 * the draft caches of a sequence must be loaded with the same length as the target. */
int spec_load_kv(spec_ctx* ctx, int32_t which, int32_t seq, const void* k /*device*/,
                 const void* v /*device*/, int32_t length);

/* Prefill: runs the target (and a draft model) over tokens[:, 0 .. P-2] appended at the
 * current length, and makes tokens[:, P-1] each sequence's last accepted token, the first
 * row of the next verify.  tokens: device int32 [batch, P], P >= 1.  Every sequence must
 * have the same length before the call.  For the MTP drafter the target's last hidden
 * state of position P-2 is kept for the head. */
int spec_prefill(spec_ctx* ctx, const int32_t* tokens /*device*/, int32_t batch, int32_t P);

/* Copies the token history of sequence `seq` (device int32 [length], positions
 * 0..length-1) for the n-gram drafter, for starts from a loaded cache prefix.  prefill,
 * set_last and accept keep the history up to date themselves. */
int spec_load_history(spec_ctx* ctx, int32_t seq, const int32_t* tokens /*device*/, int32_t length);

/* Sets each sequence's last accepted token (device int32 [batch]) without a forward, for
 * starts from a loaded cache prefix of length L: that token sits at position L.
 * prev_tok (device int32 [batch]) is the token at position L-1; a draft model's first
 * forward of every cycle recomputes its cache entry at L-1 from it, so the draft cache
 * prefix needs only L-1 valid entries.  May be NULL without a draft model.  For the MTP
 * drafter `hidden` (device float32 [batch, d_model], NULL otherwise) is the target hidden
 * state at position L-1. */
int spec_set_last(spec_ctx* ctx, const int32_t* last_tok /*device*/,
                  const int32_t* prev_tok /*device or NULL*/, const float* hidden,
                  int32_t batch);

/* ---- the cycle ----------------------------------------------------------------------- */

/* Draft k tokens per sequence (1 <= k <= max_k) from the configured drafter at one row per
 * forward.  A draft model's first forward of the cycle runs two rows, the tokens at
 * positions L-1 and L: after a cycle that accepted every draft the entry at L-1 (the last
 * draft) is missing from its cache, otherwise it is recomputed bit for bit, so no host
 * round trip is needed to tell the two apart.
 * Writes draft_tok (device int32 [batch, k]) and the truncated draft distributions q
 * (rows batch*k, row b*k + j-1 for draft j; one-hot under greedy sampling and for n-gram
 * drafts).  Draft j of sequence b is sampled with the uniform of counter
 * (j, round, b, 0).  For SPEC_DRAFT_NGRAM the call synchronizes the stream and writes to
 * *n_drafted (host, may be NULL) the largest number of drafts the lookup found for a
 * sequence (0..k); rows past a sequence's own count repeat its last found token (or its
 * last accepted token), and accept tests only that sequence's found drafts.  A batch of
 * one may then be verified at k = *n_drafted; larger batches are verified at the drafted
 * k (the row stride of draft_tok).  Other drafters write k to *n_drafted.
 * SPEC_DRAFT_MTP: the first forward of the cycle catches the MTP layer up on the positions
 * the target verified since its last draft (rows built from the target's hidden states of
 * the previous verify, or of the start), so every cycle of that drafter starts with
 * draft_step; the draft logits come from the target's LM head.
 * With a draft probability set (spec_draft_controls) a draft model / MTP sequence may stop
 * before k drafts: its draft_tok entries past the kept ones hold the placeholder id 0 (or the
 * unconfident draft that stopped it), its q rows past them are unspecified, and accept tests
 * only the kept drafts; *n_drafted is still k. */
int draft_step(spec_ctx* ctx, int32_t batch, int32_t k, uint64_t round,
               int32_t* draft_tok /*device*/, spec_probs* q /*host struct of device ptrs*/,
               int32_t* n_drafted /*host, may be NULL*/);

/* One target forward over k+1 rows per sequence: the last accepted token and draft_tok
 * (device int32 [batch, k], any source; NULL when k = 0) at positions L..L+k, appending
 * their keys and values to the cache.  Writes the truncated target distributions p (rows
 * batch*(k+1)) and, when logits_out is not NULL, the float32 logits (device
 * [batch, k+1, vocab]).  k = 0 is one step of plain decoding.  The host tracks bounds on
 * the device-side lengths; when L + k + 1 might exceed max_ctx + max_k + 2 the call
 * synchronizes the stream once to read the exact lengths, and errors with SPEC_E_RANGE if
 * the rows really do not fit.  draft_step does the same. */
int verify_step(spec_ctx* ctx, const int32_t* draft_tok /*device*/, int32_t batch, int32_t k,
                float* logits_out /*device or NULL*/, spec_probs* p /*host struct*/);

/* The accept rule per sequence.  Greedy sampler: d_j is kept iff it equals the argmax of
 * p_{j-1}; the first mismatch emits that argmax; all kept emits the argmax of p_k.
 * Otherwise d_j is kept iff u_j < p_{j-1}(d_j) / q_j(d_j) (float32 division, u_j from
 * counter (j, round, b, 1)); the first rejection emits a draw from max(0, p_{j-1} - q_j)
 * renormalized (from p_{j-1} if that is all zero), all kept emits a draw from p_k, both
 * with the uniform of counter (0, round, b, 2) walking ids in ascending order.
 * Writes n_acc (device int32 [batch], 0..k), out_tok (device int32 [batch, k+1], the first
 * n+1 entries valid: accepted drafts then the correction or bonus token), near_tie
 * (device uint8 [batch] of SPEC_FLAG_* bits, may be NULL), updates the device-side last
 * accepted token and the statistics.  A target row p_{j-1} with no entry (its logits held no
 * finite value) stops the sequence at n = j - 1 kept drafts with SPEC_FLAG_BAD_ROW and -1 as
 * its emitted token (the device-side last token becomes 0).  After a draft_step with draft
 * controls, each sequence is tested on its kept drafts only (none when they are fewer than
 * min_draft), the bonus coming from the row after them.  Must follow a verify_step with the
 * same k. */
int accept(spec_ctx* ctx, const int32_t* draft_tok /*device*/, const spec_probs* q,
           const spec_probs* p, int32_t batch, int32_t k, uint64_t round,
           int32_t* n_acc /*device*/, int32_t* out_tok /*device*/, uint8_t* near_tie);

/* Rolls every cache back to the accepted prefix: L <- L + 1 + n_acc[b] (the last accepted
 * token and its n accepted drafts stay; the emitted last token is the next cycle's first
 * row).  Must follow accept.  n_acc: device int32 [batch], each value clamped to [0, k] of
 * the cycle. */
int kv_trim(spec_ctx* ctx, const int32_t* n_acc /*device*/, int32_t batch);

/* ---- n-gram acceptance gate (host only) -------------------------------------------------
 * "Speculative decoding on Apple Silicon" (OptiQ docs), section "N-gram lookup: any model":
 * one verify pass is timed per draft length when the model loads, and each step's length
 * is chosen from how often recent drafts were accepted; with the gate off the longest
 * draft is always taken.  Reading (the page gives no formula): alpha is an exponential
 * moving average (weight 0.5, starting at 1) of accepted / attempted per step; the gate
 * picks the k in 0..n_max that maximizes (1 + alpha + ... + alpha^k) /
 * (cost[k] + k * draft_cost), costs relative to the verify at k = 0, the smallest k among
 * values within 1e-12.  k = 0: verify without drafts this step. */
typedef struct spec_gate {
  int32_t n_max;
  int32_t enabled;
  double weight;                  /* moving-average weight of the old alpha (0.5)        */
  double alpha;                   /* current acceptance estimate                          */
  double draft_cost;              /* one draft's cost relative to the k = 0 verify        */
  double cost[SPEC_MAX_K + 1];    /* verify cost at k drafts relative to k = 0            */
} spec_gate;

/* verify_cost: host double [n_max + 1] (any time unit, all > 0); draft_cost >= 0 in the
 * same unit. */
int spec_gate_init(spec_gate* g /*host*/, int32_t n_max, const double* verify_cost /*host*/,
                   double draft_cost, int32_t enabled);
/* The draft length of the next step (>= 0), or SPEC_E_INVAL for a null gate. */
int32_t spec_gate_choose(const spec_gate* g /*host*/);
/* Folds one step's accepted / attempted drafts into alpha (nothing when attempted = 0). */
int spec_gate_update(spec_gate* g /*host*/, int32_t accepted, int32_t attempted);

/* ---- adaptive draft length (host) ----------------------------------------------------
 * "Speculative decoding on Apple Silicon" (OptiQ docs), section "About depth": the heuristic
 * that raises K after a cycle whose drafts were all accepted and lowers it after a cycle with
 * a rejection.  The pages give no step sizes: K moves up by `up` and down by `down` drafts,
 * within [k_min, k_max]; a cycle that drafted nothing leaves K unchanged.  Host-only state,
 * no device work: the caller passes spec_depth_choose() as draft_step's / verify_step's k and
 * reports each cycle's accepted count. */
typedef struct spec_depth {
  int32_t k, k_min, k_max, up, down;
} spec_depth;

/* SPEC_E_INVAL unless 0 <= k_min <= k0 <= k_max <= SPEC_MAX_K and up, down >= 0. */
int spec_depth_init(spec_depth* d /*host*/, int32_t k0, int32_t k_min, int32_t k_max, int32_t up,
                    int32_t down);
/* The K of the next cycle (negative: invalid d). */
int32_t spec_depth_choose(const spec_depth* d /*host*/);
/* accepted of attempted drafts in the last cycle; SPEC_E_INVAL unless 0 <= accepted <= attempted. */
int spec_depth_update(spec_depth* d /*host*/, int32_t accepted, int32_t attempted);

/* ---- tracing ------------------------------------------------------------------------- */

/* Profiling slots: slot = kernel class + 16 * model (model 0 = target, 1 = draft); classes
 * 0 embedding gather, 1 RMSNorm, 2 QKV projection, 3 attention (chunks + combine), 4 output
 * projection + residual, 5 gate/up projection + SwiGLU, 6 down projection + residual,
 * 7 LM head, 8 truncation, 9 draft sampling, 10 accept, 11 kv trim, 12 one-launch forward. */
#define SPEC_PROF_SLOTS 32

/* enable != 0: bracket every launch of the context with HIP events on its stream, filed by
 * slot (launches then go out one by one, not as a replayed graph).  0: stop. */
int spec_profile(spec_ctx* ctx, int32_t enable);

/* While profiling, each launch of the gate/up projection slot `slot` (5 target, 21 draft)
 * goes out `reps` times back to back between its events (launches counts each): first with
 * the weights of the following reps - 1 layers, so that no launch finds its weights in a
 * cache, then the real one, which overwrites their output.  The average duration then carries
 * one dispatch delay per reps launches instead of one per launch.  SPEC_E_INVAL for another
 * slot or reps outside 1..64; reps = 1 turns it off. */
int spec_profile_repeat(spec_ctx* ctx, int32_t slot, int32_t reps);

/* Sums the recorded launches per slot: ms (host double [SPEC_PROF_SLOTS]) = total GPU time
 * between each launch's events, launches (host int64 [SPEC_PROF_SLOTS]) = launch count;
 * then forgets them.  Synchronizes the stream. */
int spec_profile_read(spec_ctx* ctx, double* ms, int64_t* launches);

/* enable != 0 (the default): draft_step and verify_step capture their launches into a HIP
 * graph on first use for a given (batch, k, buffer addresses) and replay it afterwards;
 * needs a non-default stream.  0: launch kernel by kernel. */
int spec_use_graphs(spec_ctx* ctx, int32_t enable);

/* Which projections the draft model's one- and two-row forwards take on SPEC_SCHED_STREAM
 * ("Speculative Decoding on Apple Silicon: 119% Faster...", section "The original result:
 * Qwen3-8B and a 0.6B draft": the draft runs one token at a time, so its projections move a few
 * MB for one or two rows).  enable != 0 (the default): the vector-ALU projections (one
 * workgroup per 16 weight rows, every load issued at once); 0: the MFMA weight-streaming
 * projections the target uses, rows padded to 16.  Both compute the same contract (each row's
 * results within float32 summation order of the other's); the switch exists to measure where
 * one overtakes the other.  Takes effect at the next draft_step; graphs are kept per setting.
 * Errors: SPEC_E_INVAL for a null context. */
int spec_use_gemv(spec_ctx* ctx, int32_t enable);

/* Schedule of the forwards of bf16 models over at most 16 rows (the streamed projections also
 * take 17 to 32 rows, as two launches of at most 16 rows each).
 *   SPEC_SCHED_STEP    one launch per step, one workgroup per 16-row tile of each projection;
 *   SPEC_SCHED_STREAM  (the default) one launch per step, projections streaming their weights
 *                      through an LDS ring with one workgroup per compute unit;
 *   SPEC_SCHED_FORWARD the whole forward as one persistent (cooperative) launch of the
 *                      SPEC_SCHED_STREAM steps meeting at grid barriers, the next
 *                      projection's weights streaming while a barrier is awaited; draft_step
 *                      and verify_step are then launched directly, not replayed from graphs.
 * In all three no normalization launch exists: the residual update (or the embedding) leaves
 * the float32 rows x * gain and per-16-column sums of squares of x, and the projection that
 * takes RMSNorm(x) * gain rounds (x * gain) / rms(x) to bf16 as it loads its input.  Shapes a
 * schedule does not cover (reduction lengths that are not whole 1 KB stages, head sizes other
 * than 128 or d_model above 4096 for SPEC_SCHED_FORWARD, the MTP head) fall back to the next
 * simpler one.  Schedules agree within the float tolerances, not
 * bit for bit; each is row-count invariant on its own.  Returns SPEC_E_INVAL for an unknown
 * schedule. */
#define SPEC_SCHED_STEP 0
#define SPEC_SCHED_STREAM 1
#define SPEC_SCHED_FORWARD 2
int spec_set_schedule(spec_ctx* ctx, int32_t schedule);

/* Timeline of the one-launch forward (SPEC_SCHED_FORWARD): with buf set (device, caller
 * owned, at least grid * 16 bytes), every later launch writes, per grid barrier e and
 * workgroup g, the 100 MHz constant clock at arrival and at departure to
 * buf[(e * grid + g) * 2 + {0, 1}] (unsigned 64-bit), for e < bytes / (grid * 16); e = 0 is
 * the start of the launch.  buf == NULL turns it off.  *grid (host, may be NULL) receives the
 * launch's workgroup count (0: the one-launch forward is not available). */
int spec_trace_forward(spec_ctx* ctx, void* buf /*device*/, int64_t bytes, int32_t* grid /*host*/);

/* Copies the device counters to *out (synchronizes the stream). */
int spec_get_stats(spec_ctx* ctx, spec_stats* out /*host*/);

/* Reads the current cache length of each sequence (synchronizes the stream). */
int spec_get_lengths(spec_ctx* ctx, int32_t* lengths /*host [batch]*/, int32_t batch);

/* Diagnostics: copies the start of one of the context's activation buffers, as the last
 * forward of that model left it, to dst (device, caller-owned; min(bytes, buffer size)
 * bytes, enqueued on the context stream).  which: 0 target, 1 draft model, 2 MTP layer.
 * Rows are the forward's rows (sequence-major), all float32 unless noted:
 *   SPEC_BUF_RESIDUAL   [rows, d_model] residual stream after the last layer;
 *   SPEC_BUF_NORM_INPUT [rows, d_model] the next RMSNorm input: x * gain (bf16 models) or the
 *                       normed rows (f32 models);
 *   SPEC_BUF_Q, _K      [rows, n_q_heads*head_dim], [rows, n_kv_heads*head_dim] the last
 *                       layer's q and k before RoPE (per-launch schedules);
 *   SPEC_BUF_ATTN       [rows, n_q_heads*head_dim] model dtype: the last layer's attention output;
 *   SPEC_BUF_SWIGLU     [rows, d_ffn] model dtype: the last layer's SwiGLU product;
 *   SPEC_BUF_CACHE_K,_V the whole cache, [max_batch, n_layers, n_kv_heads, capacity, head_dim]
 *                       in the model dtype, capacity = max_ctx + max_k + 2;
 *   SPEC_BUF_LOGITS     [rows, vocab] the logits of the model's last forward that kept them in
 *                       its own buffer (a verify without logits_out; the MTP head's last
 *                       forward).  A draft model's draft_step over `batch` sequences keeps the
 *                       logits of each of its forwards: forward 1 (two rows a sequence) in rows
 *                       2b and 2b + 1, forward j >= 2 in row j * batch + b; draft j (1-based) of
 *                       sequence b was drawn from row 2b + 1 (j = 1) or j * batch + b (j >= 2).
 *                       The buffer holds max(rows of one forward, (max_k + 1) * max_batch) rows
 *                       for the draft model. */
#define SPEC_BUF_RESIDUAL 0
#define SPEC_BUF_NORM_INPUT 1
#define SPEC_BUF_Q 2
#define SPEC_BUF_K 3
#define SPEC_BUF_ATTN 4
#define SPEC_BUF_SWIGLU 5
#define SPEC_BUF_CACHE_K 6
#define SPEC_BUF_CACHE_V 7
#define SPEC_BUF_LOGITS 8
int spec_debug_read(spec_ctx* ctx, int32_t which, int32_t buffer, void* dst /*device*/, size_t bytes);

/* Draft controls ("What is Speculative Decoding and How Does a Draft Model Work?", section "The
 * demo, draft model on and off with two pairings": the max draft tokens / min draft tokens /
 * draft probability settings).  The k passed to draft_step is the most drafts.  p_min in
 * [0, 1]: the draft model or MTP head stops proposing, for a sequence, at the first draft j whose
 * list gives the drawn token a probability below p_min (drafts 1 .. j-1 are kept, draft j and
 * later are not); once every sequence has stopped, the rest of the draft_step's forwards are
 * skipped on the device (their launches return at once).  Greedy lists are one-hot, so under the
 * greedy sampler p_min never stops a draft.  min_draft >= 0: a sequence whose kept drafts are
 * fewer than min_draft has none of them checked (accept emits the target's own token at row 0).
 * Both act on the next draft_step (the n-gram drafter: min_draft only).  Default 0, 0 (off).
 * Only between cycles (SPEC_E_STATE otherwise); SPEC_E_INVAL for values out of range; a
 * draft_step with p_min > 0 supports at most 64 sequences (SPEC_E_UNSUPPORTED). */
int spec_draft_controls(spec_ctx* ctx, float p_min, int32_t min_draft);

/* ---- stateless kernels (the accept workload on its own) ------------------------------ */

/* Scratch bytes spec_truncate needs for `rows` rows of `vocab` logits. */
int spec_truncate_scratch_size(int32_t rows, int32_t vocab, size_t* bytes /*host out*/);

/* Truncates `rows` rows of logits (device, dtype SPEC_DTYPE_F32 or SPEC_DTYPE_BF16, row r
 * at logits + r*row_stride elements) with sampler s into out (rows `rows`).  flags (device
 * uint8 [rows], may be NULL) receives SPEC_FLAG_TOPP_TIE / SPEC_FLAG_BAD_ROW; a bad row
 * gets count 0.  scratch: device, >= spec_truncate_scratch_size bytes. */
int spec_truncate(const void* logits /*device*/, int32_t dtype, int32_t rows, int32_t vocab,
                  int64_t row_stride, const spec_sampler* s /*host*/, spec_probs* out,
                  uint8_t* flags /*device or NULL*/, void* scratch /*device*/,
                  size_t scratch_bytes, void* stream);

/* spec_truncate for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and the
 * same results, with the partial lists in a fixed device array of SPEC_NOALLOC_SCRATCH_BYTES
 * bytes that the library holds on each GPU it runs on until the process ends.  Calls
 * spec_truncate_scratch_size would size above that limit return SPEC_E_RANGE (e.g. 1088 rows of
 * a 151936-token vocabulary need 5.6 MB).  The call allocates nothing; on its first call on a
 * device it looks up that device's copy of the array (SPEC_E_HIP if that fails).  Every call on
 * one GPU shares the array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  stream must belong to the current device. */
#define SPEC_NOALLOC_SCRATCH_BYTES (8u << 20)
int spec_truncate_noalloc(const void* logits /*device*/, int32_t dtype, int32_t rows, int32_t vocab,
                          int64_t row_stride, const spec_sampler* s /*host*/, spec_probs* out,
                          uint8_t* flags /*device or NULL*/, void* stream);

/* Draws one token per row from lists (rows = batch*per_seq; row r is slot r%per_seq + 1
 * of sequence r/per_seq) with the uniform of counter (slot, round, seq, stream_id): ids
 * walked in ascending order, first running sum above u*Z.  tokens: device int32 [rows];
 * flags: device uint8 [rows] or NULL (SPEC_FLAG_SAMPLE_TIE). */
int spec_sample(const spec_probs* lists, int32_t batch, int32_t per_seq, uint64_t seed,
                uint64_t round, int32_t stream_id, int32_t* tokens /*device*/,
                uint8_t* flags /*device or NULL*/, void* stream);

/* The accept rule of `accept` on explicit lists, without a context: q rows batch*k, p rows
 * batch*(k+1), greedy != 0 selects the greedy rule. */
int spec_accept_lists(const int32_t* draft_tok /*device*/, const spec_probs* q,
                      const spec_probs* p, int32_t batch, int32_t k, int32_t greedy,
                      uint64_t seed, uint64_t round, int32_t* n_acc /*device*/,
                      int32_t* out_tok /*device*/, uint8_t* near_tie /*device or NULL*/,
                      void* stream);

/* ---- linear-attention layer state under speculation ----------------------------------
 * "Speculative Decoding on Apple Silicon: 119% Faster...", section "Why this needed a patch to
 * mlx_lm at all": a linear-attention (Gated DeltaNet-style) layer of a hybrid model keeps one
 * fixed-size recurrent state, so a rejected draft cannot be sliced off; the state from before
 * the speculative forward is kept and the accepted tokens are run through the recurrence
 * again.  The recurrence (the gated delta rule; the pages name the layer, not the formula),
 * per head with a state S of d_v rows and d_k = 128 columns:
 *   S <- alpha S (I - beta k k^T) + beta v k^T,   o = S q.
 * One call does one cycle's state work: the first n_commit tokens (those the previous verify
 * kept: its first input and its accepted drafts) are folded into the committed state, which is
 * written back; then the next n_fwd tokens (this verify's inputs) run from it without changing
 * it and give their outputs.  A call with n_fwd = 0 only commits; n_commit = 0 only runs.
 * All buffers are device float32, token-major, caller-owned: q, k [T][n_heads][d_k],
 * v [T][n_heads][d_v], alpha, beta [T][n_heads] with T = n_commit + n_fwd (q rows below
 * n_commit are not read); state [n_heads][d_v][d_k] (in/out); out [n_fwd][n_heads][d_v].
 * q and k come normalized and alpha, beta activated, as the layer's projections leave them.
 * Returns SPEC_E_UNSUPPORTED unless d_k = 128 and d_v is a multiple of 32, SPEC_E_RANGE for
 * more than SPEC_GDN_MAX_TOKENS tokens; asynchronous on stream (errors in spec_last_error(NULL)). */
#define SPEC_GDN_MAX_TOKENS 64
typedef struct spec_gdn_shape {
  int32_t n_heads, d_k, d_v;
} spec_gdn_shape;
int spec_gdn_commit_forward(const spec_gdn_shape* shape, float* state, const float* q, const float* k,
                            const float* v, const float* alpha, const float* beta, int32_t n_commit,
                            int32_t n_fwd, float* out, void* stream);

/* n uniforms of Philox4x32-10 under key `seed`: counters ctr (device uint32 [n, 4]) ->
 * out (device float32 [n]), u = (word0 >> 8) * 2^-24. */
int spec_philox_uniforms(uint64_t seed, const uint32_t* ctr /*device*/, int32_t n,
                         float* out /*device*/, void* stream);

/* Longest-then-latest n-gram match for `batch` contexts: ctx (device int32 [batch, ld]),
 * lengths (device int32 [batch]); for each sequence, among earlier end positions e the
 * match length is the number of tokens (up to max_match) equal going backwards from e and
 * from the last token; the largest length >= n_min wins, the latest e among equals.  Writes
 * drafts (device int32 [batch, k]: the tokens after e, not past the end, then repeats of
 * the last one written or of the last context token), n_found (device int32 [batch],
 * 0..k) and match (device int32 [batch, 2]: length, e; 0, -1 when none). */
int spec_ngram_match(const int32_t* ctx /*device*/, const int32_t* lengths /*device*/,
                     int32_t batch, int32_t ld, int32_t k, int32_t n_min, int32_t max_match,
                     int32_t* drafts /*device*/, int32_t* n_found /*device*/,
                     int32_t* match /*device*/, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_H_ */
