// Kernel argument blocks and host-side launchers of the HIP library.
#pragma once

#include "common.h"

namespace spec {

// ---- truncation / sampling / accept --------------------------------------------------
struct TruncArgs {
  const void* logits;
  int64_t stride;     // elements between rows
  int vocab, rows;
  float temperature;  // <= 0: greedy
  int ksel;           // entries kept per segment: top_k, or 1 for greedy
  int nseg, seg_len;  // segments per row and their length (multiple of 8)
  uint64_t* part;     // [rows][nseg][ksel] keys, descending, 0 = empty
  uint8_t* bad;       // [rows][nseg]
  const uint32_t* skip;  // draft early stop: when set and non-zero, the launch does nothing
};

struct AcceptArgs {
  const int32_t* drafts;  // [batch, k]
  int min_draft;          // fewer drafts than this (after kcap) are not tested at all
  spec_probs q, p;        // rows batch*k and batch*(k+1)
  int batch, k, greedy;
  uint64_t seed;
  uint32_t round;
  int32_t* n_acc;         // [batch]
  int32_t* out_tok;       // [batch, k+1]
  uint8_t* near_tie;      // [batch] or null
  int32_t* last_tok;      // context state or null
  int32_t* prev_tok;
  int64_t* stats;         // 4 counters or null
  const int32_t* kcap;    // [batch] drafts found per sequence (fewer than k) or null
  int32_t* hist;          // token history [batch][hist_ld] or null: the emitted tokens are
  int hist_ld;            // appended at positions len[b]+1 .. len[b]+1+n
  const int32_t* len;
};

struct NgramArgs {
  const int32_t* ctx;
  const int32_t* lengths;  // tokens in sequence b: lengths[b] + len_add
  int batch, ld, k, n_min, max_match, len_add;
  int32_t* drafts;
  int32_t* n_found;
  int32_t* match;
};

int truncate_scratch_bytes(int rows, int vocab, size_t* bytes);
// Output row of input row r is r * out_rs.
hipError_t launch_truncate(const void* logits, int dtype, int rows, int vocab, int64_t stride,
                           const spec_sampler& s, const spec_probs& out, int out_rs, uint8_t* flags,
                           void* scratch, hipStream_t st, const uint32_t* skip = nullptr);
// Row r = (seq r / per_seq, j = r % per_seq) reads list row r * list_rs and draws with slot
// slot_base + j into tokens[seq * tok_ld + j].  The round is *rnd_ptr when rnd_ptr is not
// null (device memory, so a captured launch can be replayed for a new round), else rnd.
hipError_t launch_sample(const spec_probs& lists, int list_rs, int rows, int per_seq, int slot_base,
                         uint64_t seed, const uint32_t* rnd_ptr, uint32_t rnd, uint32_t stream_id,
                         int32_t* tokens, int tok_ld, uint8_t* flags, hipStream_t st);
// Draft controls of a draft_step (one row per sequence, rows <= 64): `kept` holds the drafts each
// sequence still proposes (k at the start); drawing draft j (slot j) from a list that gives it
// less than p_min sets kept[seq] = j - 1 for a sequence still at k >= j, and once no sequence
// proposes past draft j, *skip = 1 (the later draft forwards then do nothing).
struct DraftCtl {
  int32_t* kept;
  uint32_t* skip;
  float p_min;
};
hipError_t launch_sample_ctl(const spec_probs& lists, int list_rs, int rows, int slot, uint64_t seed,
                             const uint32_t* rnd_ptr, uint32_t stream_id, int32_t* tokens, int tok_ld,
                             const DraftCtl& ctl, hipStream_t st);
// kept[b] = k for b < batch and *skip = 0: the start of a controlled draft_step.
hipError_t launch_draft_ctl_init(int32_t* kept, int batch, int k, uint32_t* skip, hipStream_t st);
hipError_t launch_set_u32(uint32_t* p, uint32_t v, hipStream_t st);
hipError_t launch_accept(const AcceptArgs& a, hipStream_t st);
// len[b] += 1 + n_acc[b] (n_acc[b] clamped to [0, k]); a second cache length (the MTP
// layer's) is first clamped to the old len[b] + 1 when mlen is not null.
hipError_t launch_trim(int32_t* len, const int32_t* n_acc, int batch, int k, int32_t* mlen, hipStream_t st);
// One-hot lists for rows b*k + j holding drafts[b*k + j].
hipError_t launch_onehot(const int32_t* drafts, int rows, const spec_probs& q, hipStream_t st);
// Token history [batch][ld]: hist[b][pos0 + i] = src[b * src_ld + i] for i < n.
hipError_t launch_hist_write(int32_t* hist, int ld, const int32_t* src, int src_ld, int batch, int n, int pos0,
                             hipStream_t st);
// hist[b][len[b]] = last[b] and, when prev is not null, hist[b][len[b]-1] = prev[b].
hipError_t launch_hist_set_last(int32_t* hist, int ld, const int32_t* len, const int32_t* last,
                                const int32_t* prev, int batch, hipStream_t st);
hipError_t launch_philox(uint64_t seed, const uint32_t* ctr, int n, float* out, hipStream_t st);
hipError_t launch_ngram(const NgramArgs& a, hipStream_t st);

// ---- model --------------------------------------------------------------------------
// EPI_QKV_ROWS (streamed projections only): the q, k and v rows of one token side by side,
// out[m, n] for n < rows0 + 2 rows1 with row stride ld.
enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_QKV = 2, EPI_SWIGLU = 3, EPI_QKV_ROWS = 4 };

// Cache layout: [batch][n_layers][n_kv][cap][head_dim] in the model dtype.
struct CacheView {
  void* k;
  void* v;
  int n_layers, n_kv, cap, hd;
};

// Rows of a forward: row m belongs to sequence m / mseq at position
// len[m / mseq] + pos_off + m % mseq.
struct RowMap {
  int M, mseq;
  const int32_t* len;
  int pos_off;
};

struct GemmArgs {
  const void* w[3];   // weight matrices [rows_i, K]; EPI_QKV uses three, EPI_SWIGLU two
  int rows[3];
  int K;
  const void* x;      // [M, K] model dtype (GEMM input as stored)
  // RMSNorm input (bf16 path): when ss_in is set, x holds the float32 rows r * g of residual
  // rows r and gain g, and the GEMM input row m is bf16((r * g) / sqrt(mean + eps)), mean =
  // (the np_in partial sums of squares ss_in[m * ss_ld + 0 .. np_in-1], added in order) / K
  const float* ss_in;
  int np_in, ss_ld;
  float eps;
  float* ss_out;      // EPI_RESID: partial sums of squares of the updated rows, one per block
  void* y_out;        // EPI_RESID (bf16 models, may be null): [M, ld] float32 updated rows * y_gain
  const void* y_gain;
  RowMap rm;
  // outputs
  float* out;         // EPI_STORE / EPI_RESID: [M, ld]
  int ld;
  void* h;            // EPI_SWIGLU: [M, rows0] model dtype
  float* q_stage;     // EPI_QKV: [M, rows0] raw q
  float* k_stage;     // EPI_QKV: [M, rows1] raw k
  CacheView cache;    // EPI_QKV: values written at their positions
  int layer;
};

struct AttnArgs {
  const float* q_stage;
  const float* k_stage;
  CacheView cache;
  int layer;
  RowMap rm;
  int n_q;
  const float2* rope;  // [cap][hd/2] cos, sin
  float scale;
  float* part;         // [M*n_q][nchunk][hd+2]
  int nchunk;
  int ngrid;           // chunks launched (0: nchunk); covers every position the rows reach
  void* out;           // combine: [M, n_q*hd] model dtype
  const uint32_t* skip;  // draft early stop: when set and non-zero, the launch does nothing
  // bf16, head_dim 128: launches with at most ATTN_FEW_ROWS query rows per kv head run their
  // chunks on the vector ALUs (attn_chunk_few_kernel) instead of 16-row MFMA tiles.  Set per
  // model, so that all its forwards at those row counts take the same path.
  int few;
};

constexpr int ATTN_FEW_ROWS = 4;

// Linear-attention (gated delta rule) state: gdn.hip.  Token-major rows: q, k [T][n_heads][128],
// v [T][n_heads][d_v], alpha, beta [T][n_heads] with T = n_commit + n_fwd; state
// [n_heads][d_v][128]; out [n_fwd][n_heads][d_v].  The first n_commit tokens are folded into
// the state, which is written back; the next n_fwd run from it (unchanged) and give out.
constexpr int GDN_DK = 128;
constexpr int GDN_MAX_TOKENS = 64;
struct GdnArgs {
  float* state;
  const float* q;
  const float* k;
  const float* v;
  const float* alpha;
  const float* beta;
  float* out;
  int n_heads, d_v;
  int n_commit, n_fwd;
};
hipError_t gdn_init();
hipError_t launch_gdn(const GdnArgs& a, hipStream_t st);

constexpr int ATTN_CHUNK = 64;
constexpr int ATTN_MAX_CHUNKS = 256;  // contexts up to 16384 positions
constexpr int ATTN_ROWS_MAX = 96;  // (tokens per sequence) x (q heads per kv head)

hipError_t launch_rope_table(float2* table, int cap, int hd, float theta, hipStream_t st);
// y (bf16 models, may be null): also writes the float32 rows * gain, the input of the first
// projection before its 1/rms.
hipError_t launch_embed(int dtype, const void* E, int d, int vocab, const int32_t* first,
                        int first_ld, const int32_t* rest, int rest_ld, int M, int mseq, float* x,
                        float* ss, int ss_ld, void* y, const void* gain, hipStream_t st);
hipError_t launch_rmsnorm(int dtype, const float* x, const void* g, float eps, int M, int d,
                          void* y, hipStream_t st);
hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t st);
// y[m, k] = x[m, k] * gain[k] in float32 for M rows of K (bf16 models): the input of a
// projection of RMSNorm(x) when the producer of x did not leave it.
hipError_t launch_gain_rows(const float* x, const void* gain, int M, int K, void* y, hipStream_t st);
hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st);
hipError_t launch_fill(void* p, size_t bytes, hipStream_t st);
hipError_t launch_copy_rows(const int32_t* src, int src_ld, int32_t* dst, int n, hipStream_t st);
size_t attention_lds_bytes(int R, int hd);
hipError_t attention_set_lds_limit();
hipError_t launch_kv_load(int dtype, const void* k, const void* v, CacheView c, int seq, int length,
                          hipStream_t st);
hipError_t launch_set_len(int32_t* len, int seq, int value, hipStream_t st);
hipError_t launch_add_len(int32_t* len, int batch, int delta, hipStream_t st);
// dst[b] = src[b] + add
hipError_t launch_len_from(int32_t* dst, const int32_t* src, int batch, int add, hipStream_t st);

// Multi-token-prediction input rows (m = b * R + i, M = batch * R): the concatenation of
// RMSNorm(h, norm_h) and RMSNorm(E[token], norm_e), rounded to the model dtype.
// h row = h + b * h_ss + i * h_rs (float32 [d]); token = tok[b * tok_ld + (tok_pos ? tok_pos[b] : 0) + i].
struct MtpInArgs {
  const float* h;
  int64_t h_ss, h_rs;
  const int32_t* tok;
  int tok_ld;
  const int32_t* tok_pos;
  const void* embed;
  const void* norm_h;
  const void* norm_e;
  float eps;
  int d, R, M, vocab;
  void* out;  // [M][2d] model dtype
};
hipError_t launch_mtp_input(int dtype, const MtpInArgs& a, hipStream_t st);
// Per sequence b, copies residual row b * R + r and its sum-of-squares partials (ss_ld floats)
// to row b of x1 / ss1, where r = len[b] - mlen[b] (clamped to 0..R-1) when mlen is not null,
// else 0.
hipError_t launch_gather_last(const float* x, const float* ss, int ss_ld, int d, int R, const int32_t* len,
                              const int32_t* mlen, int batch, float* x1, float* ss1, hipStream_t st);
// dst[b * dst_ss + i * d + e] = src[b * src_ss + i * d + e] for i < R, e < d.
hipError_t launch_copy_rows_f32(const float* src, int64_t src_ss, int R, int d, int batch, float* dst,
                                int64_t dst_ss, hipStream_t st);

// ---- weight-streaming projections (bf16 models, M <= 16 rows) -------------------------
// out[m, n] = sum_k W[n, k] x[m, k] with W streamed through an LDS ring by one workgroup per
// compute unit (see stream.hip).  Epilogues as GemmArgs, and so is the RMSNorm input: with
// ss_in set, x holds the float32 rows r * g of residual rows r and the input row m is
// bf16((r * g) / sqrt(mean + eps)), the mean from the np_in partials ss_in[m * ss_ld + 0 ..]
// added in order.  EPI_RESID adds into out (row stride ld) and leaves, when set,
// ss_out[m * ss_ld + u] = the sum of squares of the 16 updated columns of unit u, and y_out =
// float32 updated rows * y_gain (the next projection's input before its 1/rms).
struct StreamArgs {
  // EPI_QKV / EPI_QKV_ROWS: W_q, W_k, W_v; EPI_SWIGLU: W_gate, W_up; else W.  Separate
  // members, not an array: an indexed member would move the block to scratch memory.
  const void* w0;
  const void* w1;
  const void* w2;
  // fp8 weights (wbytes 1): OCP e4m3 codes, the weight of row r being code * wNs[r]
  const float* w0s;
  const float* w1s;
  const float* w2s;
  int wbytes;         // 2: bf16 weights, 1: fp8 weights with row scales
  int rows0, rows1, rows2;
  int K, nunits;      // nunits: row tiles of 16 (EPI_SWIGLU: gate/up tile pairs)
  const void* x;      // [M, K] bf16 input rows, or float32 rows r * g with ss_in set
  const float* ss_in; // RMSNorm input: partial sums of squares of the residual rows
  int np_in, ss_ld;
  float eps;
  int M;
  float* out;         // EPI_STORE / EPI_RESID: [M, ld]
  int ld;
  float* ss_out;      // EPI_RESID
  void* y_out;        // EPI_RESID: [M, ld] float32 updated rows * y_gain
  const void* y_gain;
  void* h;            // EPI_SWIGLU: [M, rows0] bf16
  float* q_stage;     // EPI_QKV
  float* k_stage;
  CacheView cache;
  int layer;
  RowMap rm;
  const uint32_t* skip;  // draft early stop: when set and non-zero, the launch does nothing
  // the forward's row of this launch's row 0 (launches of more than 16 rows run as passes of at
  // most 16): the value rows' cache positions follow it
  int row0;
  // EPI_QKV, per-launch projections: when > 0, the chunk count of the attention launch that
  // follows (grid nchunk x n_kv x batch), whose cached rows of this layer the workgroups with
  // one unit fewer than the others touch before they end (a pre-read, nothing is written)
  int pf_nchunk;
};
// Whether M rows and reduction length K are covered (M <= 32: more than 16 rows run as two
// launches, rows 0..15 and 16..M-1, each streaming the weights).  bf16 weights: K in whole
// stages (1024; 512 for SwiGLU), normalized inputs only for K in {1024, 2048, 3072, 4096, 5120}.  fp8 weights
// (wbytes 1): stages of 2048 (1024 for SwiGLU), resident inputs for K in {2048, 4096}, streamed
// inputs for the residual epilogue, and at most units_per_wg * tiles * 16 <= 1024 row scales
// per workgroup.
bool stream_supported(int M, int K, int epi, bool norm, int wbytes = 2, int units_per_wg = 1);
size_t stream_lds_bytes();
hipError_t stream_init();  // per device: LDS limit of the kernels
hipError_t launch_stream_gemm(int epi, const StreamArgs& a, int grid, hipStream_t st);

// ---- vector-ALU projections of one or two rows (gemv.hip) ----------------------------
// The streamed projections' arguments and epilogues, for M <= 2 rows and bf16 weights: RMSNorm
// inputs (ss_in set, at most 128 partials per row) for QKV and the vocabulary projection with K
// in {1024, 2048, 4096} and gate/up with K in {1024, 2048}; plain inputs for the residual
// projections with K in {1024, 2048, 3072, 3584, 4096}.  One workgroup per unit of 16 rows
// (a.nunits).
bool gemv_supported(int M, int K, int epi, bool norm, int wbytes);
hipError_t launch_gemv(int epi, const StreamArgs& a, hipStream_t st);

// ---- one persistent launch per forward (bf16 models, M <= 16 rows) ------------------
// The rows, positions and buffers of forward(); x, y, ss, q/k staging, attention partials and
// outputs and the SwiGLU product are the model's workspace buffers.  layers is a device copy
// of the layer table.  sync: forward_sync_bytes(batch, n_kv) of device memory, zero before the first
// launch (its last word is a sticky error flag: non-zero once a barrier has timed out).
struct FwdArgs {
  const spec_layer_weights* layers;
  int n_layers, d, n_q, n_kv, ffn, vocab, q_dim, kv_dim;
  float eps, scale;
  const void* embed;
  const void* lm_head;
  const void* final_norm;
  int M, mseq, pos_off;
  const int32_t* len;
  const int32_t* first;
  int first_ld;
  const int32_t* rest;
  int rest_ld;
  CacheView cache;
  const float2* rope;
  float* x;       // [M][d] residual rows
  float* y;       // [M][d] residual rows * the next norm's gain
  float* ss;      // [M][ss_ld] sum-of-squares partials
  int ss_ld;
  float* qkv;     // [M][q_dim + 2 kv_dim] raw q, k, v rows
  float* part;    // [M * n_q][nchunk][hd + 2]
  int nchunk;
  void* attn;     // [M][q_dim] bf16
  void* h;        // [M][ffn] bf16
  float* logits;  // [M][vocab] or null
  unsigned* sync;
  // optional timeline: barrier e of workgroup g writes the constant-rate clock when the
  // workgroup arrives and when it leaves to trace[(e * grid + g) * 2 + {0, 1}] (e < trace_cap)
  unsigned long long* trace;
  int trace_cap;
  const uint32_t* skip;  // draft early stop: when set and non-zero, the launch does nothing
};
bool forward_supported(int M, int mseq, int d, int n_q, int n_kv, int hd, int ffn, int vocab);
// bytes of the one-launch forward's barrier words (eight group counters, a top counter, a
// release word, the error word at byte forward_error_offset()); the same for any batch and
// n_kv, which the signature keeps for per-sequence words
size_t forward_sync_bytes(int batch, int n_kv);
constexpr size_t forward_error_offset() { return 10 * 32 * 4; }
// per device: LDS limits; *grid = workgroups of one launch (one per compute unit, a multiple
// of 8), 0 when the launch cannot be co-resident
hipError_t forward_init(int* grid);
hipError_t launch_forward(const FwdArgs& a, int grid, hipStream_t st);

}  // namespace spec
