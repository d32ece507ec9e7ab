// Host side of the C ABI: validation, workspace carving, the forward sequence of each
// model, and the draft / verify / accept / trim state machine.  No device allocation.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"

using namespace spec;

namespace {

thread_local std::string g_init_error = "no error";

// Rows per sequence of one prefill forward; also bounded by the kernels' row limits.
constexpr int PREFILL_ROWS = 16;
constexpr int GEMM_MAX_ROWS_BF16 = 64;
constexpr int GEMM_MAX_ROWS_F32 = 32;
constexpr int STREAM_MAX_ROWS = 16;  // fp8-weight models run the streamed projections only

struct Model {
  int mi = 0;  // 0 target, 1 draft (profiling slot offset 16 * mi)
  spec_model_desc d{};
  std::vector<spec_layer_weights> layers;
  std::vector<spec_layer_scales> scales;  // fp8 weights: row scales of each layer
  bool fp8 = false;                       // SPEC_WEIGHTS_FP8_ROW
  bool present = false;
  // one- and two-row forwards on the vector-ALU projections (the draft model: all its draft_step
  // forwards take them, so its rows never depend on the row count)
  bool gemv = false;
  int q_dim = 0, kv_dim = 0, mseq_max = 0, Mmax = 0, nchunk = 0;
  int logit_rows = 0;  // rows of `logits`: Mmax, or for the draft model (max_k + 1) per sequence
  size_t act = 4;
  CacheView cache{};
  float* x = nullptr;
  // the input of the next projection of an RMSNorm, float32: f32 models the normed rows; bf16
  // models rows * gain, which the projection scales by 1/rms and rounds to bf16 as it loads them
  void* xn = nullptr;
  float* qst = nullptr;
  float* kst = nullptr;
  void* attn = nullptr;
  void* h = nullptr;
  float* logits = nullptr;
  float* part = nullptr;
  float* ss = nullptr;  // [Mmax][d/16] partial sums of squares of the residual rows
  float* qkv = nullptr; // [Mmax][q_dim + 2 kv_dim] raw q, k, v rows (one-launch forward)
  spec_layer_weights* dev_layers = nullptr;  // device copy of the layer table (one-launch forward)
  float2* rope = nullptr;
  // set while a controlled draft_step is enqueued: the launches of this model's forwards then
  // do nothing once the word is non-zero (every sequence stopped proposing)
  const uint32_t* skip = nullptr;
};

// IDLE: nothing to decode from yet; READY: a last token is set, the caches are trimmed;
// DRAFTED / VERIFIED / ACCEPTED: inside a cycle.
enum Phase { IDLE = 0, READY = 1, DRAFTED = 2, VERIFIED = 3, ACCEPTED = 4 };

enum ProfClass {
  PROF_EMBED = 0, PROF_NORM = 1, PROF_QKV = 2, PROF_ATTN = 3, PROF_OPROJ = 4, PROF_GATEUP = 5,
  PROF_DOWN = 6, PROF_LMHEAD = 7, PROF_TRUNC = 8, PROF_SAMPLE = 9, PROF_ACCEPT = 10, PROF_TRIM = 11,
  PROF_FORWARD = 12
};

struct ProfRec {
  int slot;
  hipEvent_t a, b;
  int reps;  // back-to-back launches between the two events
};

// A captured launch sequence and the arguments it was captured with.
struct GraphEntry {
  int kind;  // 0 verify, 1 draft
  int batch, k;
  const void* ptrs[8];
  hipGraphExec_t exec = nullptr;
};

}  // namespace

struct spec_ctx {
  spec_config cfg{};
  Model target, draft, mtp;
  hipStream_t stream = nullptr;
  int32_t* len = nullptr;       // [max_batch] context length L per sequence
  int32_t* last_tok = nullptr;  // [max_batch] token at position L
  int32_t* prev_tok = nullptr;  // [max_batch] token at position L-1
  int64_t* stats = nullptr;     // 4 counters
  int32_t* hist = nullptr;      // [max_batch][hist_ld] tokens at positions 0..L
  int hist_ld = 0;
  int32_t* ndraft = nullptr;    // [max_batch] drafts the n-gram lookup found
  int32_t* match = nullptr;     // [max_batch][2] n-gram match length and end
  bool ngram_cycle = false;     // this cycle's drafts came from the n-gram lookup
  // draft controls (spec_draft_controls): the draft-probability threshold and the fewest drafts
  // worth checking; the draft model / MTP drafter's kept counts live in ndraft
  float p_min = 0.0f;
  int min_draft = 0;
  bool ctl_cycle = false;       // this cycle's draft_step ran with the controls
  uint32_t* dskip = nullptr;    // non-zero once no sequence proposes further drafts
  // MTP drafter: its cache length, the target hidden rows it catches up from, the gathered
  // last row and its partials, the concatenated input rows
  int32_t* mtp_len = nullptr;
  float* mtp_h = nullptr;       // [max_batch][max_k+1][d]
  float* x1 = nullptr;          // [max_batch][d]
  float* ss1 = nullptr;         // [max_batch][d/16+1]
  void* mtp_in = nullptr;       // [rows][2d] model dtype
  int mtp_rows = 1;             // rows of the next catch-up (previous cycle's k + 1)
  // schedule of bf16 forwards over few rows (SPEC_SCHED_*) and the grid of the streamed
  // projections (one workgroup per compute unit)
  int sched = SPEC_SCHED_STREAM;
  int ncu = 0;
  int fgrid = 0;            // workgroups of the one-launch forward (0: not available)
  unsigned* fsync = nullptr;  // its barrier words
  bool barrier_failed = false;  // a synchronizing call found the sticky barrier error word set
  unsigned long long* ftrace = nullptr;  // optional barrier timeline (spec_trace_forward)
  int ftrace_cap = 0;
  void* trunc = nullptr;
  size_t trunc_bytes = 0;
  int cap = 0;
  // host bookkeeping: every sequence's L lies in [len_lo, len_hi]
  int len_lo = 0, len_hi = 0;
  // attention chunks launched in the current draft_step / verify_step (0 outside them: the
  // whole capacity): enough for every position the call's rows reach, so that chunks past the
  // length are not launched; part of the graph key
  int attn_nch = 0;
  bool started = false;
  Phase phase = IDLE;
  int phase_k = -1, phase_batch = -1;
  uint32_t* round_dev = nullptr;  // the cycle's round, read by the draft sampling kernels
  // launch profiling (events around every launch; graphs are bypassed while it is on)
  bool prof = false;
  int prof_rep_slot = -1, prof_reps = 1;  // spec_profile_repeat
  hipEvent_t prof_start = nullptr;
  std::vector<hipEvent_t> ev_free;
  std::vector<ProfRec> recs;
  // graph replay of draft_step / verify_step
  bool graphs = true;
  std::vector<GraphEntry> gcache;
  std::string err = "no error";

  ~spec_ctx() {
    for (auto& g : gcache)
      if (g.exec) (void)hipGraphExecDestroy(g.exec);
    for (auto& r : recs) {
      (void)hipEventDestroy(r.a);
      (void)hipEventDestroy(r.b);
    }
    for (auto e : ev_free) (void)hipEventDestroy(e);
  }
};

namespace {

int fail(spec_ctx* c, int code, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
int fail(spec_ctx* c, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c) c->err = buf;
  else g_init_error = buf;
  return code;
}

#define HIPCHK(ctx, expr)                                                                      \
  do {                                                                                         \
    hipError_t e_ = (expr);                                                                    \
    if (e_ != hipSuccess) return fail(ctx, SPEC_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

hipError_t take_event(spec_ctx* c, hipEvent_t* e) {
  if (!c->ev_free.empty()) {
    *e = c->ev_free.back();
    c->ev_free.pop_back();
    return hipSuccess;
  }
  return hipEventCreate(e);
}

// Enqueue a launch; with profiling on, bracket it with events filed under `slot`.
#define LAUNCH(ctx, slot, expr)                                            \
  do {                                                                     \
    hipEvent_t ea_ = nullptr, eb_ = nullptr;                               \
    if ((ctx)->prof) {                                                     \
      HIPCHK(ctx, take_event(ctx, &ea_));                                  \
      HIPCHK(ctx, hipEventRecord(ea_, (ctx)->stream));                     \
    }                                                                      \
    HIPCHK(ctx, expr);                                                     \
    if ((ctx)->prof) {                                                     \
      HIPCHK(ctx, take_event(ctx, &eb_));                                  \
      HIPCHK(ctx, hipEventRecord(eb_, (ctx)->stream));                     \
      (ctx)->recs.push_back(ProfRec{(slot), ea_, eb_, 1});                 \
    }                                                                      \
  } while (0)

// LAUNCH for a launch that may be repeated under spec_profile_repeat: fn(r) issues repeat r
// of reps (r = reps - 1 is the real one).
#define LAUNCH_REP(ctx, slot, fn)                                                          \
  do {                                                                                     \
    hipEvent_t ea_ = nullptr, eb_ = nullptr;                                               \
    const int reps_ = ((ctx)->prof && (slot) == (ctx)->prof_rep_slot) ? (ctx)->prof_reps : 1; \
    if ((ctx)->prof) {                                                                     \
      HIPCHK(ctx, take_event(ctx, &ea_));                                                  \
      HIPCHK(ctx, hipEventRecord(ea_, (ctx)->stream));                                     \
    }                                                                                      \
    for (int r_ = 0; r_ < reps_; ++r_) HIPCHK(ctx, fn(r_, reps_));                         \
    if ((ctx)->prof) {                                                                     \
      HIPCHK(ctx, take_event(ctx, &eb_));                                                  \
      HIPCHK(ctx, hipEventRecord(eb_, (ctx)->stream));                                     \
      (ctx)->recs.push_back(ProfRec{(slot), ea_, eb_, reps_});                             \
    }                                                                                      \
  } while (0)

// Layer of repeat r of reps of layer l's launch: the others first, l itself last.
inline int rep_layer(int l, int r, int reps, int n_layers) { return (l + reps - 1 - r) % n_layers; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Bump carving of the workspace; with base == nullptr it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return base ? (T*)(base + o) : nullptr;
  }
};

int row_cap(const spec_model_desc& m) {
  if (m.weights == SPEC_WEIGHTS_FP8_ROW) return STREAM_MAX_ROWS;
  return m.dtype == SPEC_DTYPE_BF16 ? GEMM_MAX_ROWS_BF16 : GEMM_MAX_ROWS_F32;
}

int validate_model(const spec_model_desc& m, const char* name, int max_k, int max_batch, bool need_w) {
  if (m.n_layers < 1 || m.d_model < 16 || m.n_q_heads < 1 || m.n_kv_heads < 1 || m.head_dim < 2 ||
      m.d_ffn < 16 || m.vocab < 2)
    return fail(nullptr, SPEC_E_INVAL, "%s: non-positive shape", name);
  if (m.dtype != SPEC_DTYPE_F32 && m.dtype != SPEC_DTYPE_BF16)
    return fail(nullptr, SPEC_E_INVAL, "%s: dtype %d", name, m.dtype);
  if (m.head_dim != 32 && m.head_dim != 64 && m.head_dim != 128)
    return fail(nullptr, SPEC_E_UNSUPPORTED, "%s: head_dim %d (32, 64 or 128)", name, m.head_dim);
  if (m.weights != SPEC_WEIGHTS_NATIVE && m.weights != SPEC_WEIGHTS_FP8_ROW)
    return fail(nullptr, SPEC_E_INVAL, "%s: weights %d", name, m.weights);
  if (m.weights == SPEC_WEIGHTS_FP8_ROW && m.dtype != SPEC_DTYPE_BF16)
    return fail(nullptr, SPEC_E_UNSUPPORTED, "%s: fp8 weights need a bf16 model", name);
  if (m.n_q_heads % m.n_kv_heads)
    return fail(nullptr, SPEC_E_INVAL, "%s: n_q_heads not a multiple of n_kv_heads", name);
  const int q = m.n_q_heads * m.head_dim, kv = m.n_kv_heads * m.head_dim;
  if (m.dtype == SPEC_DTYPE_BF16) {
    if (m.d_model % 32 || m.d_ffn % 32 || q % 32 || kv % 16 || m.vocab % 16)
      return fail(nullptr, SPEC_E_UNSUPPORTED,
                  "%s: bf16 projections need in-features %% 32 == 0 and out-features %% 16 == 0", name);
  }
  const int G = m.n_q_heads / m.n_kv_heads;
  if ((max_k + 1) * G > ATTN_ROWS_MAX)
    return fail(nullptr, SPEC_E_UNSUPPORTED, "%s: (max_k+1) * q-heads-per-kv-head > %d", name, ATTN_ROWS_MAX);
  const int rmax = row_cap(m);
  if (max_batch * (max_k + 1) > rmax)
    return fail(nullptr, SPEC_E_UNSUPPORTED, "%s: max_batch*(max_k+1) > %d rows", name, rmax);
  if (!(m.rms_eps >= 0.0f) || !(m.rope_theta > 0.0f))
    return fail(nullptr, SPEC_E_INVAL, "%s: rms_eps / rope_theta", name);
  if (need_w) {
    if (!m.embed || !m.lm_head || !m.final_norm || !m.layers)
      return fail(nullptr, SPEC_E_INVAL, "%s: null weight pointer", name);
    for (int l = 0; l < m.n_layers; ++l) {
      const spec_layer_weights& w = m.layers[l];
      if (!w.attn_norm || !w.wq || !w.wk || !w.wv || !w.wo || !w.ffn_norm || !w.wg || !w.wu || !w.wd)
        return fail(nullptr, SPEC_E_INVAL, "%s: null weight pointer in layer %d", name, l);
    }
    if (m.weights == SPEC_WEIGHTS_FP8_ROW) {
      if (m.lm_head == m.embed)
        return fail(nullptr, SPEC_E_UNSUPPORTED, "%s: fp8 weights need an untied LM head", name);
      if (!m.lm_head_scale || !m.layer_scales) return fail(nullptr, SPEC_E_INVAL, "%s: null scale pointer", name);
      for (int l = 0; l < m.n_layers; ++l) {
        const spec_layer_scales& w = m.layer_scales[l];
        if (!w.wq || !w.wk || !w.wv || !w.wo || !w.wg || !w.wu || !w.wd)
          return fail(nullptr, SPEC_E_INVAL, "%s: null scale pointer in layer %d", name, l);
      }
    }
  }
  return SPEC_OK;
}

int validate_sampler(const spec_sampler& s) {
  if (!(s.temperature == s.temperature)) return SPEC_E_INVAL;
  if (s.temperature > 0.0f) {
    if (s.top_k < 1 || s.top_k > SPEC_TOPK_MAX) return SPEC_E_UNSUPPORTED;
    if (!(s.top_p > 0.0f) || !(s.top_p <= 1.0f)) return SPEC_E_INVAL;
  }
  return SPEC_OK;
}

int max_rows_per_seq(const spec_model_desc& m, int max_k, int max_batch) {
  const int G = m.n_q_heads / m.n_kv_heads;
  const int rmax = row_cap(m);
  int r = std::max(max_k + 1, PREFILL_ROWS);
  r = std::min(r, ATTN_ROWS_MAX / G);
  r = std::min(r, rmax / max_batch);
  return std::max(r, max_k + 1);
}

void carve_model(Model& m, Carver& cv, int B, int cap, int logit_rows = 0) {
  const spec_model_desc& d = m.d;
  m.act = d.dtype == SPEC_DTYPE_BF16 ? 2 : 4;
  m.q_dim = d.n_q_heads * d.head_dim;
  m.kv_dim = d.n_kv_heads * d.head_dim;
  m.Mmax = B * m.mseq_max;
  m.nchunk = (cap + ATTN_CHUNK - 1) / ATTN_CHUNK;
  const size_t cache_elems = (size_t)B * d.n_layers * d.n_kv_heads * cap * d.head_dim;
  m.cache.k = cv.take<void>(cache_elems * m.act);
  m.cache.v = cv.take<void>(cache_elems * m.act);
  m.cache.n_layers = d.n_layers;
  m.cache.n_kv = d.n_kv_heads;
  m.cache.cap = cap;
  m.cache.hd = d.head_dim;
  m.x = cv.take<float>((size_t)m.Mmax * d.d_model * 4);
  m.xn = cv.take<void>((size_t)m.Mmax * d.d_model * 4);
  m.qst = cv.take<float>((size_t)m.Mmax * m.q_dim * 4);
  m.kst = cv.take<float>((size_t)m.Mmax * m.kv_dim * 4);
  m.attn = cv.take<void>((size_t)m.Mmax * m.q_dim * m.act);
  m.h = cv.take<void>((size_t)m.Mmax * d.d_ffn * m.act);
  m.logit_rows = std::max(m.Mmax, logit_rows);
  m.logits = cv.take<float>((size_t)m.logit_rows * d.vocab * 4);
  m.part = cv.take<float>((size_t)m.Mmax * d.n_q_heads * m.nchunk * (d.head_dim + 2) * 4);
  m.ss = cv.take<float>((size_t)m.Mmax * (d.d_model / 16 + 1) * 4);
  m.qkv = cv.take<float>((size_t)m.Mmax * (m.q_dim + 2 * m.kv_dim) * 4);
  m.dev_layers = cv.take<spec_layer_weights>((size_t)d.n_layers * sizeof(spec_layer_weights));
  m.rope = cv.take<float2>((size_t)cap * (d.head_dim / 2) * sizeof(float2));
}

// Layout shared by spec_workspace_size and spec_init.
size_t layout(spec_ctx* c, void* ws) {
  Carver cv(ws);
  const spec_config& g = c->cfg;
  const int B = g.max_batch;
  c->cap = g.max_ctx + g.max_k + 2;
  c->len = cv.take<int32_t>(B * 4);
  c->last_tok = cv.take<int32_t>(B * 4);
  c->prev_tok = cv.take<int32_t>(B * 4);
  c->stats = cv.take<int64_t>(4 * 8);
  c->round_dev = cv.take<uint32_t>(4);
  c->dskip = cv.take<uint32_t>(4);
  c->hist_ld = c->cap + 1;
  c->hist = cv.take<int32_t>((size_t)B * c->hist_ld * 4);
  c->ndraft = cv.take<int32_t>(B * 4);
  c->match = cv.take<int32_t>(B * 8);
  c->fsync = cv.take<unsigned>(forward_sync_bytes(B, std::max(g.target.n_kv_heads, c->draft.present ? g.draft.n_kv_heads : 0)));
  c->target.mseq_max = max_rows_per_seq(c->target.d, g.max_k, B);
  carve_model(c->target, cv, B, c->cap);
  if (c->draft.present) {
    c->draft.mseq_max = std::max(2, max_rows_per_seq(c->draft.d, 1, B));
    // a draft_step keeps every forward's logits: forward 1 in rows 0 .. 2B-1, forward j >= 2
    // in rows jB .. jB + B - 1
    carve_model(c->draft, cv, B, c->cap, (g.max_k + 1) * B);
  }
  if (c->mtp.present) {
    const int d = c->mtp.d.d_model;
    c->mtp.mseq_max = c->target.mseq_max;
    carve_model(c->mtp, cv, B, c->cap);
    c->mtp_len = cv.take<int32_t>(B * 4);
    c->mtp_h = cv.take<float>((size_t)B * (g.max_k + 1) * d * 4);
    c->x1 = cv.take<float>((size_t)B * d * 4);
    c->ss1 = cv.take<float>((size_t)B * (d / 16 + 1) * 4);
    c->mtp_in = cv.take<void>((size_t)c->mtp.Mmax * 2 * d * c->mtp.act);
  }
  size_t tb = 0;
  const int rows = std::max(std::max(c->target.Mmax, c->draft.present ? c->draft.Mmax : 0),
                            c->mtp.present ? c->mtp.Mmax : 0);
  truncate_scratch_bytes(rows, g.target.vocab, &tb);
  c->trunc_bytes = tb;
  c->trunc = cv.take<void>(tb);
  return cv.off;
}

int check_config(spec_ctx* c, const spec_config* cfg) {
  if (!cfg) return fail(nullptr, SPEC_E_INVAL, "null config");
  c->cfg = *cfg;
  const spec_config& g = c->cfg;
  if (g.max_batch < 1 || g.max_ctx < 1 || g.max_k < 0 || g.max_k > SPEC_MAX_K)
    return fail(nullptr, SPEC_E_INVAL, "max_batch / max_ctx / max_k out of range");
  if (g.max_ctx + g.max_k + 2 > ATTN_CHUNK * ATTN_MAX_CHUNKS)
    return fail(nullptr, SPEC_E_UNSUPPORTED, "max_ctx + max_k + 2 > %d", ATTN_CHUNK * ATTN_MAX_CHUNKS);
  int rc = validate_sampler(g.sampler);
  if (rc) return fail(nullptr, rc, "sampler: temperature / top_k (1..%d) / top_p", SPEC_TOPK_MAX);
  const int maxk = std::max(g.max_k, 1);
  rc = validate_model(g.target, "target", maxk, g.max_batch, false);
  if (rc) return rc;
  if (g.target.weights == SPEC_WEIGHTS_FP8_ROW && g.draft_kind == SPEC_DRAFT_MTP)
    return fail(nullptr, SPEC_E_UNSUPPORTED, "fp8 target weights with the MTP drafter");
  c->target.d = g.target;
  c->target.fp8 = g.target.weights == SPEC_WEIGHTS_FP8_ROW;
  c->target.present = true;
  c->target.mi = 0;
  if (g.draft_kind == SPEC_DRAFT_MODEL) {
    rc = validate_model(g.draft, "draft", 1, g.max_batch, false);
    if (rc) return rc;
    if (g.draft.vocab != g.target.vocab)
      return fail(nullptr, SPEC_E_INVAL, "draft vocab %d != target vocab %d", g.draft.vocab, g.target.vocab);
    c->draft.d = g.draft;
    c->draft.fp8 = g.draft.weights == SPEC_WEIGHTS_FP8_ROW;
    c->draft.present = true;
    c->draft.mi = 1;
    c->draft.gemv = true;
  } else if (g.draft_kind == SPEC_DRAFT_MTP) {
    // one extra decoder layer at the target's widths, its own final norm, the target's
    // embedding and LM head
    c->mtp.d = g.target;
    c->mtp.d.n_layers = 1;
    c->mtp.d.final_norm = g.mtp.final_norm;
    c->mtp.d.layers = nullptr;
    c->mtp.d.weights = SPEC_WEIGHTS_NATIVE;
    c->mtp.d.layer_scales = nullptr;
    c->mtp.present = true;
    c->mtp.mi = 1;
  } else if (g.draft_kind == SPEC_DRAFT_NGRAM) {
    if (g.ngram.n_min < 1 || g.ngram.max_match < g.ngram.n_min)
      return fail(nullptr, SPEC_E_INVAL, "ngram: need 1 <= n_min <= max_match");
  } else if (g.draft_kind != SPEC_DRAFT_NONE) {
    return fail(nullptr, SPEC_E_INVAL, "draft kind %d", g.draft_kind);
  }
  if (g.sampler.temperature > 0.0f && g.sampler.top_k > g.target.vocab)
    return fail(nullptr, SPEC_E_INVAL, "top_k > vocab");
  size_t tb = 0;
  if (truncate_scratch_bytes(1, g.target.vocab, &tb))
    return fail(nullptr, SPEC_E_UNSUPPORTED, "vocab %d too large for the truncation kernels", g.target.vocab);
  return SPEC_OK;
}

spec_probs offset_rows(const spec_probs& p, int rows) {
  spec_probs o = p;
  o.ids += (int64_t)rows * p.cap;
  o.probs += (int64_t)rows * p.cap;
  o.count += rows;
  return o;
}

int check_probs(spec_ctx* c, const spec_probs* p, const char* name, int need_cap) {
  if (!p || !p->ids || !p->probs || !p->count)
    return fail(c, SPEC_E_INVAL, "%s: null spec_probs buffer", name);
  if (p->cap < need_cap) return fail(c, SPEC_E_INVAL, "%s: cap %d < %d", name, p->cap, need_cap);
  return SPEC_OK;
}

int list_cap(const spec_sampler& s) { return s.temperature > 0.0f ? s.top_k : 1; }

// RMSNorm input of a projection.  bf16 models have no normalization pass: the projection reads
// the float32 rows x * gain and the row's np sum-of-squares partials ss, and rounds
// (x * gain) / rms(x) to bf16 as it loads them; `ready` says that the producer of x already
// left x * gain in m.xn, otherwise one small kernel writes it.  f32 models run the plain
// RMSNorm kernel.
int norm_input(spec_ctx* c, Model& m, GemmArgs& g, int M, const float* x, const float* ss, int np,
               const void* gain, bool ready) {
  const spec_model_desc& d = m.d;
  const int P = 16 * m.mi;
  if (d.dtype != SPEC_DTYPE_BF16) {
    LAUNCH(c, P + PROF_NORM, launch_rmsnorm(d.dtype, x, gain, d.rms_eps, M, d.d_model, m.xn, c->stream));
    g.x = m.xn;
    return SPEC_OK;
  }
  // bf16: the projection reads x * gain and the partials of x; the residual epilogue (or the
  // embedding) that produced x normally left those rows in m.xn already
  if (!ready) LAUNCH(c, P + PROF_NORM, launch_gain_rows(x, gain, M, d.d_model, m.xn, c->stream));
  g.x = m.xn;
  g.ss_in = ss;
  g.np_in = np;
  g.ss_ld = d.d_model / 16 + 1;
  g.eps = d.rms_eps;
  return SPEC_OK;
}

// Whether the attention of m runs its chunks on the vector ALUs: the draft model with head_dim
// 128 and at most two q heads per kv head, so that its draft_step forwards (one or two rows)
// have at most ATTN_FEW_ROWS query rows per kv head and all take the same path (a row's
// results then do not depend on the row count; prefill chunks of more rows take the MFMA
// kernel).
bool attn_few(spec_ctx* c, const Model& m) {
  const spec_model_desc& d = m.d;
  return &m == &c->draft && d.dtype == SPEC_DTYPE_BF16 && d.head_dim == 128 &&
         2 * (d.n_q_heads / d.n_kv_heads) <= ATTN_FEW_ROWS;
}

// Attention chunks to launch for m: those the current draft_step / verify_step can reach (the
// MTP head keeps its whole capacity: its length follows the target's by its own rule).
int attn_grid(spec_ctx* c, const Model& m) {
  return (c->attn_nch > 0 && &m != &c->mtp) ? std::min(c->attn_nch, m.nchunk) : m.nchunk;
}

// Whether the forwards of m over M rows run on the weight-streaming projections: bf16,
// at most 16 rows, reduction lengths in whole stages (normalized inputs: d in {1024, 2048,
// 3072, 4096, 5120}).  The MTP head keeps the per-row-tile kernels: its input projection leaves no
// gain-multiplied rows.
bool stream_shapes(spec_ctx* c, const Model& m, int M) {
  const spec_model_desc& d = m.d;
  if (c->ncu < 1 || (m.q_dim + 2 * m.kv_dim) % 16 || d.d_ffn % 16 || d.vocab % 16 || d.d_model % 16) return false;
  const int wb = m.fp8 ? 1 : 2;
  // units per workgroup (the fp8 kernels keep that many tiles of row scales in LDS)
  auto upw = [&](int nunits) {
    const int g = std::min(c->ncu, nunits);
    return (nunits + g - 1) / g;
  };
  return stream_supported(M, d.d_model, EPI_QKV, true, wb, upw((m.q_dim + 2 * m.kv_dim) / 16)) &&
         stream_supported(M, d.d_model, EPI_SWIGLU, true, wb, upw(d.d_ffn / 16)) &&
         stream_supported(M, m.q_dim, EPI_RESID, false, wb, upw(d.d_model / 16)) &&
         stream_supported(M, d.d_ffn, EPI_RESID, false, wb, upw(d.d_model / 16)) &&
         stream_supported(M, d.d_model, EPI_STORE, true, wb, upw(d.vocab / 16));
}

// Whether the streamed-schedule forwards of m over M rows take the vector-ALU projections: a
// model flagged for them (the draft), bf16 weights, at most 2 rows, and every projection shape
// covered (RMSNorm inputs with at most 128 partials).
bool use_gemv(const Model& m, int M) {
  const spec_model_desc& d = m.d;
  if (!m.gemv || m.fp8 || d.dtype != SPEC_DTYPE_BF16 || d.d_model / 16 > 128) return false;
  return gemv_supported(M, d.d_model, EPI_QKV, true, 2) && gemv_supported(M, m.q_dim, EPI_RESID, false, 2) &&
         gemv_supported(M, d.d_model, EPI_SWIGLU, true, 2) && gemv_supported(M, d.d_ffn, EPI_RESID, false, 2);
}

// fp8-weight models take these kernels under every schedule (no other kernel decodes fp8).
bool use_stream(spec_ctx* c, const Model& m, int M) {
  const spec_model_desc& d = m.d;
  if (d.dtype != SPEC_DTYPE_BF16 || &m == &c->mtp || (!m.fp8 && c->sched != SPEC_SCHED_STREAM)) return false;
  return stream_shapes(c, m, M);
}

// The decoder layers of m on the streamed projections over the M rows in m.x (np
// sum-of-squares partials per row in m.ss).
int run_layers_stream(spec_ctx* c, Model& m, int M, RowMap rm, int np) {
  const spec_model_desc& d = m.d;
  const int P = 16 * m.mi;
  const int grid = c->ncu;
  const int ss_ld = d.d_model / 16 + 1;
  const int wb = m.fp8 ? 1 : 2;
  const spec_layer_scales no_scales{};
  const bool gv = use_gemv(m, M);
  auto proj = [&](int epi, const StreamArgs& a) {
    return gv ? launch_gemv(epi, a, c->stream) : launch_stream_gemm(epi, a, grid, c->stream);
  };
  for (int l = 0; l < d.n_layers; ++l) {
    const spec_layer_weights& w = m.layers[l];
    const spec_layer_scales& sc = m.fp8 ? m.scales[l] : no_scales;
    StreamArgs g{};
    g.skip = m.skip;
    g.w0 = w.wq;
    g.w1 = w.wk;
    g.w2 = w.wv;
    g.w0s = sc.wq;
    g.w1s = sc.wk;
    g.w2s = sc.wv;
    g.wbytes = wb;
    g.rows0 = m.q_dim;
    g.rows1 = m.kv_dim;
    g.rows2 = m.kv_dim;
    g.K = d.d_model;
    g.nunits = (m.q_dim + 2 * m.kv_dim) / 16;
    g.x = m.xn;
    g.ss_in = m.ss;
    g.np_in = np;
    g.ss_ld = ss_ld;
    g.eps = d.rms_eps;
    g.M = M;
    g.q_stage = m.qst;
    g.k_stage = m.kst;
    g.cache = m.cache;
    g.layer = l;
    g.rm = rm;
    g.pf_nchunk = attn_grid(c, m);  // the attention launch below: grid (chunks, n_kv, batch)
    LAUNCH(c, P + PROF_QKV, proj(EPI_QKV, g));
    AttnArgs at{};
    at.skip = m.skip;
    at.q_stage = m.qst;
    at.k_stage = m.kst;
    at.cache = m.cache;
    at.layer = l;
    at.rm = rm;
    at.n_q = d.n_q_heads;
    at.rope = m.rope;
    at.scale = 1.0f / sqrtf((float)d.head_dim);
    at.part = m.part;
    at.nchunk = m.nchunk;
    at.ngrid = attn_grid(c, m);
    at.few = attn_few(c, m);
    at.out = m.attn;
    LAUNCH(c, P + PROF_ATTN, launch_attention(d.dtype, at, c->stream));
    StreamArgs o{};
    o.skip = m.skip;
    o.w0 = w.wo;
    o.w0s = sc.wo;
    o.wbytes = wb;
    o.rows0 = d.d_model;
    o.K = m.q_dim;
    o.nunits = d.d_model / 16;
    o.x = m.attn;
    o.M = M;
    o.out = m.x;
    o.ld = d.d_model;
    o.ss_out = m.ss;
    o.ss_ld = ss_ld;
    o.y_out = m.xn;
    o.y_gain = w.ffn_norm;
    LAUNCH(c, P + PROF_OPROJ, proj(EPI_RESID, o));
    np = d.d_model / 16;
    StreamArgs gu{};
    gu.skip = m.skip;
    gu.w0 = w.wg;
    gu.w1 = w.wu;
    gu.w0s = sc.wg;
    gu.w1s = sc.wu;
    gu.wbytes = wb;
    gu.rows0 = d.d_ffn;
    gu.K = d.d_model;
    gu.nunits = d.d_ffn / 16;
    gu.x = m.xn;
    gu.ss_in = m.ss;
    gu.np_in = np;
    gu.ss_ld = ss_ld;
    gu.eps = d.rms_eps;
    gu.M = M;
    gu.h = m.h;
    auto gu_rep = [&](int r, int reps) {
      StreamArgs g2 = gu;
      const int lr = rep_layer(l, r, reps, d.n_layers);
      g2.w0 = m.layers[lr].wg;
      g2.w1 = m.layers[lr].wu;
      if (m.fp8) {
        g2.w0s = m.scales[lr].wg;
        g2.w1s = m.scales[lr].wu;
      }
      return proj(EPI_SWIGLU, g2);
    };
    LAUNCH_REP(c, P + PROF_GATEUP, gu_rep);
    StreamArgs dn{};
    dn.skip = m.skip;
    dn.w0 = w.wd;
    dn.w0s = sc.wd;
    dn.wbytes = wb;
    dn.rows0 = d.d_model;
    dn.K = d.d_ffn;
    dn.nunits = d.d_model / 16;
    dn.x = m.h;
    dn.M = M;
    dn.out = m.x;
    dn.ld = d.d_model;
    dn.ss_out = m.ss;
    dn.ss_ld = ss_ld;
    dn.y_out = m.xn;
    dn.y_gain = l + 1 < d.n_layers ? m.layers[l + 1].attn_norm : d.final_norm;
    LAUNCH(c, P + PROF_DOWN, proj(EPI_RESID, dn));
  }
  return SPEC_OK;
}

// The decoder layers of m over the M rows already in m.x (np sum-of-squares partials per
// row in m.ss for bf16 models), rows placed by rm.
int run_layers(spec_ctx* c, Model& m, int M, RowMap rm, int np) {
  if (use_stream(c, m, M)) return run_layers_stream(c, m, M, rm, np);
  if (m.fp8) return fail(c, SPEC_E_UNSUPPORTED, "fp8 weights over %d rows", M);
  const spec_model_desc& d = m.d;
  const hipStream_t st = c->stream;
  const int dt = d.dtype;
  const int P = 16 * m.mi;
  const bool fused = dt == SPEC_DTYPE_BF16;
  const int ss_ld = d.d_model / 16 + 1;
  for (int l = 0; l < d.n_layers; ++l) {
    const spec_layer_weights& w = m.layers[l];
    GemmArgs g{};
    g.w[0] = w.wq;
    g.w[1] = w.wk;
    g.w[2] = w.wv;
    g.rows[0] = m.q_dim;
    g.rows[1] = m.kv_dim;
    g.rows[2] = m.kv_dim;
    g.K = d.d_model;
    if (norm_input(c, m, g, M, m.x, m.ss, np, w.attn_norm, true)) return SPEC_E_HIP;
    g.rm = rm;
    g.q_stage = m.qst;
    g.k_stage = m.kst;
    g.cache = m.cache;
    g.layer = l;
    LAUNCH(c, P + PROF_QKV, launch_gemm(dt, EPI_QKV, g, st));
    AttnArgs a{};
    a.skip = m.skip;
    a.q_stage = m.qst;
    a.k_stage = m.kst;
    a.cache = m.cache;
    a.layer = l;
    a.rm = rm;
    a.n_q = d.n_q_heads;
    a.rope = m.rope;
    a.scale = 1.0f / sqrtf((float)d.head_dim);
    a.part = m.part;
    a.nchunk = m.nchunk;
    a.ngrid = attn_grid(c, m);
    a.out = m.attn;
    a.few = attn_few(c, m);
    LAUNCH(c, P + PROF_ATTN, launch_attention(dt, a, st));
    GemmArgs o{};
    o.w[0] = w.wo;
    o.rows[0] = d.d_model;
    o.K = m.q_dim;
    o.x = m.attn;
    o.rm = rm;
    o.out = m.x;
    o.ld = d.d_model;
    o.ss_out = fused ? m.ss : nullptr;
    o.ss_ld = ss_ld;
    o.y_out = fused ? m.xn : nullptr;
    o.y_gain = w.ffn_norm;
    LAUNCH(c, P + PROF_OPROJ, launch_gemm(dt, EPI_RESID, o, st));
    np = d.d_model / 16;
    GemmArgs gu{};
    gu.w[0] = w.wg;
    gu.w[1] = w.wu;
    gu.rows[0] = d.d_ffn;
    gu.K = d.d_model;
    if (norm_input(c, m, gu, M, m.x, m.ss, np, w.ffn_norm, true)) return SPEC_E_HIP;
    gu.rm = rm;
    gu.h = m.h;
    auto gu_rep = [&](int r, int reps) {
      GemmArgs g2 = gu;
      g2.w[0] = m.layers[rep_layer(l, r, reps, d.n_layers)].wg;
      g2.w[1] = m.layers[rep_layer(l, r, reps, d.n_layers)].wu;
      return launch_gemm(dt, EPI_SWIGLU, g2, st);
    };
    LAUNCH_REP(c, P + PROF_GATEUP, gu_rep);
    GemmArgs dn{};
    dn.w[0] = w.wd;
    dn.rows[0] = d.d_model;
    dn.K = d.d_ffn;
    dn.x = m.h;
    dn.rm = rm;
    dn.out = m.x;
    dn.ld = d.d_model;
    dn.ss_out = fused ? m.ss : nullptr;
    dn.ss_ld = ss_ld;
    dn.y_out = fused ? m.xn : nullptr;
    dn.y_gain = l + 1 < d.n_layers ? m.layers[l + 1].attn_norm : d.final_norm;
    LAUNCH(c, P + PROF_DOWN, launch_gemm(dt, EPI_RESID, dn, st));
  }
  return SPEC_OK;
}

// Final RMSNorm and vocabulary projection of M residual rows x (ss: their partials, np per
// row) into logits [M, vocab].
int run_head(spec_ctx* c, Model& m, int M, RowMap rm, const float* x, const float* ss, int np, float* logits) {
  const spec_model_desc& d = m.d;
  if (use_stream(c, m, M) && x == m.x && ss == m.ss) {
    StreamArgs lm{};
    lm.skip = m.skip;
    lm.w0 = d.lm_head;
    lm.w0s = m.fp8 ? d.lm_head_scale : nullptr;
    lm.wbytes = m.fp8 ? 1 : 2;
    lm.rows0 = d.vocab;
    lm.K = d.d_model;
    lm.nunits = d.vocab / 16;
    lm.x = m.xn;
    lm.ss_in = ss;
    lm.np_in = np;
    lm.ss_ld = d.d_model / 16 + 1;
    lm.eps = d.rms_eps;
    lm.M = M;
    lm.out = logits;
    lm.ld = d.vocab;
    // the draft's one or two rows take the vector-ALU kernel: a workgroup per 16 vocabulary rows
    // (9496 at 151936), many resident per CU, instead of the ring's per-unit cross-wavefront
    // reduction every 32 KB stage (0.6B tied table: 52.4 -> 48.1 us by events)
    const bool gv = use_gemv(m, M) && gemv_supported(M, d.d_model, EPI_STORE, true, 2);
    LAUNCH(c, 16 * m.mi + PROF_LMHEAD,
           gv ? launch_gemv(EPI_STORE, lm, c->stream) : launch_stream_gemm(EPI_STORE, lm, c->ncu, c->stream));
    return SPEC_OK;
  }
  if (m.fp8) return fail(c, SPEC_E_UNSUPPORTED, "fp8 LM head outside the streamed projections");
  GemmArgs lm{};
  lm.w[0] = d.lm_head;
  lm.rows[0] = d.vocab;
  lm.K = d.d_model;
  // rows of m.x come with bf16(x * final gain) from the last layer's residual epilogue
  if (norm_input(c, m, lm, M, x, ss, np, d.final_norm, x == m.x)) return SPEC_E_HIP;
  lm.rm = rm;
  lm.out = logits;
  lm.ld = d.vocab;
  LAUNCH(c, 16 * m.mi + PROF_LMHEAD, launch_gemm(d.dtype, EPI_STORE, lm, c->stream));
  return SPEC_OK;
}

// Whether the forward of m over B x mseq rows runs as one persistent launch.
bool use_forward(spec_ctx* c, const Model& m, int B, int mseq) {
  const spec_model_desc& d = m.d;
  if (c->sched != SPEC_SCHED_FORWARD || c->fgrid < 8 || d.dtype != SPEC_DTYPE_BF16 || &m == &c->mtp || m.fp8)
    return false;
  if (B * mseq > c->fgrid) return false;
  return forward_supported(B * mseq, mseq, d.d_model, d.n_q_heads, d.n_kv_heads, d.head_dim, d.d_ffn, d.vocab);
}

int forward_one_launch(spec_ctx* c, Model& m, int B, int mseq, const int32_t* first, int first_ld,
                       const int32_t* rest, int rest_ld, int pos_off, float* logits) {
  const spec_model_desc& d = m.d;
  FwdArgs a{};
  a.skip = m.skip;
  a.layers = m.dev_layers;
  a.n_layers = d.n_layers;
  a.d = d.d_model;
  a.n_q = d.n_q_heads;
  a.n_kv = d.n_kv_heads;
  a.ffn = d.d_ffn;
  a.vocab = d.vocab;
  a.q_dim = m.q_dim;
  a.kv_dim = m.kv_dim;
  a.eps = d.rms_eps;
  a.scale = 1.0f / sqrtf((float)d.head_dim);
  a.embed = d.embed;
  a.lm_head = d.lm_head;
  a.final_norm = d.final_norm;
  a.M = B * mseq;
  a.mseq = mseq;
  a.pos_off = pos_off;
  a.len = c->len;
  a.first = first;
  a.first_ld = first_ld;
  a.rest = rest ? rest : first;
  a.rest_ld = rest_ld;
  a.cache = m.cache;
  a.rope = m.rope;
  a.x = m.x;
  a.y = (float*)m.xn;
  a.ss = m.ss;
  a.ss_ld = d.d_model / 16 + 1;
  a.qkv = m.qkv;
  a.part = m.part;
  a.nchunk = m.nchunk;
  a.attn = m.attn;
  a.h = m.h;
  a.logits = logits;
  a.sync = c->fsync;
  a.trace = c->ftrace;
  a.trace_cap = c->ftrace_cap;
  LAUNCH(c, 16 * m.mi + PROF_FORWARD, launch_forward(a, c->fgrid, c->stream));
  return SPEC_OK;
}

// One forward of model m over M = B*mseq rows; rows' tokens come from first/rest (see
// launch_embed) at positions len + pos_off + i.  Logits go to `logits` when non-null.
int forward(spec_ctx* c, Model& m, int B, int mseq, const int32_t* first, int first_ld,
            const int32_t* rest, int rest_ld, int pos_off, float* logits) {
  if (use_forward(c, m, B, mseq)) return forward_one_launch(c, m, B, mseq, first, first_ld, rest, rest_ld, pos_off, logits);
  const spec_model_desc& d = m.d;
  const int M = B * mseq;
  const bool fused = d.dtype == SPEC_DTYPE_BF16;
  const int ss_ld = d.d_model / 16 + 1;
  RowMap rm{M, mseq, c->len, pos_off};
  LAUNCH(c, 16 * m.mi + PROF_EMBED, launch_embed(d.dtype, d.embed, d.d_model, d.vocab, first, first_ld, rest, rest_ld,
                                                 M, mseq, m.x, fused ? m.ss : nullptr, ss_ld, fused ? m.xn : nullptr,
                                                 m.layers[0].attn_norm, c->stream));
  int rc = run_layers(c, m, M, rm, 1);
  if (rc) return rc;
  if (logits) return run_head(c, m, M, rm, m.x, m.ss, d.d_model / 16, logits);
  return SPEC_OK;
}

// The MTP layer over R rows per sequence at positions mtp_len[b] + pos_off + i: input rows
// [RMSNorm(h); RMSNorm(E[token])] projected by w_proj into the residual stream, then the
// layer.  h row (b, i) = h + b * h_ss + i * d; token (b, i) = tok[b * tok_ld + (tok_pos ?
// tok_pos[b] : 0) + i].
int mtp_layer(spec_ctx* c, int B, int R, const float* h, int64_t h_ss, const int32_t* tok, int tok_ld,
              const int32_t* tok_pos, int pos_off) {
  Model& m = c->mtp;
  const spec_model_desc& d = m.d;
  const spec_mtp_desc& w = c->cfg.mtp;
  const int M = B * R;
  MtpInArgs in{};
  in.h = h;
  in.h_ss = h_ss;
  in.h_rs = d.d_model;
  in.tok = tok;
  in.tok_ld = tok_ld;
  in.tok_pos = tok_pos;
  in.embed = d.embed;
  in.norm_h = w.norm_h;
  in.norm_e = w.norm_e;
  in.eps = d.rms_eps;
  in.d = d.d_model;
  in.R = R;
  in.M = M;
  in.vocab = d.vocab;
  in.out = c->mtp_in;
  LAUNCH(c, 16 * m.mi + PROF_EMBED, launch_mtp_input(d.dtype, in, c->stream));
  // the projection lands in a zeroed residual stream: 0 + v is v exactly, and the residual
  // epilogue leaves the sum-of-squares partials the layer's first norm reads
  HIPCHK(c, launch_fill(m.x, (size_t)M * d.d_model * 4, c->stream));
  const bool fused = d.dtype == SPEC_DTYPE_BF16;
  GemmArgs g{};
  g.w[0] = w.w_proj;
  g.rows[0] = d.d_model;
  g.K = 2 * d.d_model;
  g.x = c->mtp_in;
  RowMap rm{M, R, c->mtp_len, pos_off};
  g.rm = rm;
  g.out = m.x;
  g.ld = d.d_model;
  g.ss_out = fused ? m.ss : nullptr;
  g.ss_ld = d.d_model / 16 + 1;
  g.y_out = fused ? m.xn : nullptr;
  g.y_gain = m.layers[0].attn_norm;
  LAUNCH(c, 16 * m.mi + PROF_EMBED, launch_gemm(d.dtype, EPI_RESID, g, c->stream));
  return run_layers(c, m, M, rm, d.d_model / 16);
}

int need_ctx(spec_ctx* c) { return c ? SPEC_OK : SPEC_E_INVAL; }

// After a call that synchronized the stream: the one-launch forward's sticky error word.  Once
// it is set every result since the failed barrier is invalid, and every later cycle call of
// the context fails.
int read_barrier_error(spec_ctx* c) {
  if (c->barrier_failed) return fail(c, SPEC_E_HIP, "a grid barrier of the one-launch forward timed out");
  unsigned err = 0;
  HIPCHK(c, hipMemcpyAsync(&err, (const char*)c->fsync + forward_error_offset(), sizeof err, hipMemcpyDeviceToHost,
                           c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  if (err) {
    c->barrier_failed = true;
    return fail(c, SPEC_E_HIP, "a grid barrier of the one-launch forward timed out");
  }
  return SPEC_OK;
}
int cycle_usable(spec_ctx* c) {
  if (c->barrier_failed) return fail(c, SPEC_E_HIP, "a grid barrier of the one-launch forward timed out earlier");
  return SPEC_OK;
}

// The host only knows bounds on the device lengths (an accept may keep 0..k drafts).  When
// the upper bound leaves less than `need` free cache slots, read the exact lengths of the
// first `batch` sequences (this synchronizes the stream) and tighten the bounds.
int ensure_room(spec_ctx* c, int batch, int need) {
  if (c->len_hi + need <= c->cap) return SPEC_OK;
  std::vector<int32_t> h(batch);
  HIPCHK(c, hipMemcpyAsync(h.data(), c->len, sizeof(int32_t) * batch, hipMemcpyDeviceToHost, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  int lo = h[0], hi = h[0];
  for (int b = 1; b < batch; ++b) {
    lo = std::min(lo, h[b]);
    hi = std::max(hi, h[b]);
  }
  c->len_lo = lo;
  c->len_hi = hi;
  if (int rc = read_barrier_error(c)) return rc;
  if (c->len_hi + need > c->cap) return fail(c, SPEC_E_RANGE, "context would overflow the cache");
  return SPEC_OK;
}


// The kernels of one draft_step: k forwards of the draft model at one row (two rows for
// the first: the tokens at L-1 and L), each followed by truncation and a sampled draft.
// Draws draft j of every sequence from its list row j - 1; with a draft-probability threshold
// the controlled kernel also stops the sequences whose draft falls below it.
int enqueue_draft_sample(spec_ctx* c, Model& m, int batch, int k, int j, int32_t* draft_tok, const spec_probs& q) {
  const int P = 16 * m.mi;
  if (c->p_min > 0.0f) {
    LAUNCH(c, P + PROF_SAMPLE, launch_sample_ctl(offset_rows(q, j - 1), k, batch, j, c->cfg.seed, c->round_dev,
                                                 STREAM_DRAFT, draft_tok + (j - 1), k,
                                                 DraftCtl{c->ndraft, c->dskip, c->p_min}, c->stream));
  } else {
    LAUNCH(c, P + PROF_SAMPLE, launch_sample(offset_rows(q, j - 1), k, batch, 1, j, c->cfg.seed, c->round_dev,
                                             0u, STREAM_DRAFT, draft_tok + (j - 1), k, nullptr, c->stream));
  }
  return SPEC_OK;
}

// With a draft-probability threshold the draft_step starts by setting every sequence's kept
// count to k and clearing the stop word, and the model's launches check that word.
struct DraftSkipScope {
  Model& m;
  DraftSkipScope(spec_ctx* c, Model& mm) : m(mm) { m.skip = c->p_min > 0.0f ? c->dskip : nullptr; }
  ~DraftSkipScope() { m.skip = nullptr; }
};

int enqueue_draft(spec_ctx* c, int batch, int k, int32_t* draft_tok, const spec_probs& q) {
  Model& m = c->draft;
  const spec_sampler& s = c->cfg.sampler;
  const int V = m.d.vocab;
  const int P = 16 * m.mi;
  if (c->p_min > 0.0f) HIPCHK(c, launch_draft_ctl_init(c->ndraft, batch, k, c->dskip, c->stream));
  DraftSkipScope scope(c, m);
  // each forward keeps its logits in rows of its own (forward 1: 0 .. 2 batch - 1; forward j:
  // j batch .. j batch + batch - 1), which the context's logits buffer holds up to max_k
  for (int j = 1; j <= k; ++j) {
    int rc;
    if (j == 1) {
      rc = forward(c, m, batch, 2, c->prev_tok, 1, c->last_tok, 1, -1, m.logits);
      if (rc) return rc;
      LAUNCH(c, P + PROF_TRUNC, launch_truncate(m.logits + V, SPEC_DTYPE_F32, batch, V, 2 * (int64_t)V, s, q, k,
                                                nullptr, c->trunc, c->stream, m.skip));
    } else {
      float* lg = m.logits + (size_t)j * batch * V;
      rc = forward(c, m, batch, 1, draft_tok + (j - 2), k, nullptr, 0, j - 1, lg);
      if (rc) return rc;
      LAUNCH(c, P + PROF_TRUNC, launch_truncate(lg, SPEC_DTYPE_F32, batch, V, V, s, offset_rows(q, j - 1), k,
                                                nullptr, c->trunc, c->stream, m.skip));
    }
    rc = enqueue_draft_sample(c, m, batch, k, j, draft_tok, q);
    if (rc) return rc;
  }
  return SPEC_OK;
}

// The kernels of one MTP draft_step.  The first forward catches the head up on the target:
// R rows at positions mtp_len[b] .. from the target hidden states of the previous verify (or
// the start) and the tokens of the history; the logits come from the row at position L.
// Every later draft is one row fed with the head's own last hidden state and the previous
// draft.
int enqueue_draft_mtp(spec_ctx* c, int batch, int k, int32_t* draft_tok, const spec_probs& q) {
  Model& m = c->mtp;
  const spec_sampler& s = c->cfg.sampler;
  const int V = m.d.vocab, d = m.d.d_model;
  const int P = 16 * m.mi;
  const int ss_ld = d / 16 + 1;
  const bool fused = m.d.dtype == SPEC_DTYPE_BF16;
  const int R = c->mtp_rows;
  const int64_t h_ss = (int64_t)(c->cfg.max_k + 1) * d;
  if (c->p_min > 0.0f) HIPCHK(c, launch_draft_ctl_init(c->ndraft, batch, k, c->dskip, c->stream));
  DraftSkipScope scope(c, m);
  for (int j = 1; j <= k; ++j) {
    int rc;
    if (j == 1) {
      rc = mtp_layer(c, batch, R, c->mtp_h, h_ss, c->hist, c->hist_ld, c->mtp_len, 0);
      if (rc) return rc;
      HIPCHK(c, launch_gather_last(m.x, fused ? m.ss : nullptr, ss_ld, d, R, c->len, c->mtp_len, batch, c->x1,
                                   c->ss1, c->stream));
      // the head's cache now holds positions up to L
      HIPCHK(c, launch_len_from(c->mtp_len, c->len, batch, 1, c->stream));
    } else {
      rc = mtp_layer(c, batch, 1, c->x1, d, draft_tok + (j - 2), k, nullptr, j - 2);
      if (rc) return rc;
      HIPCHK(c, launch_gather_last(m.x, fused ? m.ss : nullptr, ss_ld, d, 1, c->len, nullptr, batch, c->x1, c->ss1,
                                   c->stream));
    }
    RowMap rm{batch, 1, c->mtp_len, 0};
    rc = run_head(c, m, batch, rm, c->x1, c->ss1, d / 16, m.logits);
    if (rc) return rc;
    LAUNCH(c, P + PROF_TRUNC, launch_truncate(m.logits, SPEC_DTYPE_F32, batch, V, V, s, offset_rows(q, j - 1), k,
                                              nullptr, c->trunc, c->stream, m.skip));
    rc = enqueue_draft_sample(c, m, batch, k, j, draft_tok, q);
    if (rc) return rc;
  }
  return SPEC_OK;
}

// The kernels of one n-gram draft_step: the longest-then-latest match in each sequence's
// history (positions 0..L) and one-hot draft lists.
int enqueue_draft_ngram(spec_ctx* c, int batch, int k, int32_t* draft_tok, const spec_probs& q) {
  NgramArgs a{c->hist, c->len, batch, c->hist_ld, k, c->cfg.ngram.n_min, c->cfg.ngram.max_match, 1,
              draft_tok, c->ndraft, c->match};
  LAUNCH(c, 16 + PROF_SAMPLE, launch_ngram(a, c->stream));
  LAUNCH(c, 16 + PROF_SAMPLE, launch_onehot(draft_tok, batch * k, q, c->stream));
  return SPEC_OK;
}

// The kernels of one verify_step: the target forward over k+1 rows and the truncation.
int enqueue_verify(spec_ctx* c, const int32_t* draft_tok, int batch, int k, float* logits_out,
                   const spec_probs& p) {
  Model& m = c->target;
  const int V = m.d.vocab;
  float* lg = logits_out ? logits_out : m.logits;
  int rc = forward(c, m, batch, k + 1, c->last_tok, 1, draft_tok, k, 0, lg);
  if (rc) return rc;
  // the MTP head catches up next cycle from these hidden states (positions L .. L+k)
  if (c->mtp.present)
    HIPCHK(c, launch_copy_rows_f32(m.x, (int64_t)(k + 1) * m.d.d_model, k + 1, m.d.d_model, batch, c->mtp_h,
                                   (int64_t)(c->cfg.max_k + 1) * m.d.d_model, c->stream));
  LAUNCH(c, PROF_TRUNC, launch_truncate(lg, SPEC_DTYPE_F32, batch * (k + 1), V, V, c->cfg.sampler, p, 1, nullptr,
                                        c->trunc, c->stream));
  return SPEC_OK;
}

// The attention chunks a draft_step / verify_step launches: positions below len_hi + need (the
// rows it appends), rounded up to 4 chunks (256 positions), so that a growing context takes a
// new graph every 256 positions; restored to the whole capacity when the call returns.
struct NchScope {
  spec_ctx* c;
  NchScope(spec_ctx* cc, int need) : c(cc) {
    const int n = (c->len_hi + need + 1) / ATTN_CHUNK + 1;
    c->attn_nch = (n + 3) / 4 * 4;
  }
  ~NchScope() { c->attn_nch = 0; }
};

// Runs `enqueue` directly, or through a captured graph: the first call with a given
// (kind, batch, k, buffer addresses) captures the launches on the context stream, later
// calls replay them.  Every kernel reads lengths and the round from device memory, so a
// replay computes exactly what a direct enqueue would.
template <typename F>
int run_graphed(spec_ctx* c, int kind, int batch, int k, const void* const key[8], F enqueue) {
  // cooperative launches stay out of captured graphs
  if (c->prof || !c->graphs || c->stream == nullptr || c->sched == SPEC_SCHED_FORWARD) return enqueue();
  // graphs are kept per schedule and per projection choice of the draft model
  const int gkind = kind + 16 * c->sched + 64 * (c->draft.gemv ? 1 : 0);
  for (auto& g : c->gcache) {
    if (g.kind == gkind && g.batch == batch && g.k == k && !memcmp(g.ptrs, key, sizeof g.ptrs)) {
      HIPCHK(c, hipGraphLaunch(g.exec, c->stream));
      return SPEC_OK;
    }
  }
  HIPCHK(c, hipStreamBeginCapture(c->stream, hipStreamCaptureModeThreadLocal));
  int rc = enqueue();
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamEndCapture(c->stream, &graph);
  if (rc) {
    if (graph) (void)hipGraphDestroy(graph);
    return rc;
  }
  if (e != hipSuccess) return fail(c, SPEC_E_HIP, "graph capture: %s", hipGetErrorString(e));
  GraphEntry g;
  g.kind = gkind;
  g.batch = batch;
  g.k = k;
  memcpy(g.ptrs, key, sizeof g.ptrs);
  e = hipGraphInstantiate(&g.exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (e != hipSuccess) return fail(c, SPEC_E_HIP, "graph instantiate: %s", hipGetErrorString(e));
  if (c->gcache.size() >= 32) {
    (void)hipGraphExecDestroy(c->gcache.front().exec);
    c->gcache.erase(c->gcache.begin());
  }
  c->gcache.push_back(g);
  HIPCHK(c, hipGraphLaunch(g.exec, c->stream));
  return SPEC_OK;
}

}  // namespace

// =====================================================================================
extern "C" {

int spec_workspace_size(const spec_config* cfg, size_t* bytes) {
  if (!bytes) return fail(nullptr, SPEC_E_INVAL, "null bytes");
  spec_ctx tmp;
  int rc = check_config(&tmp, cfg);
  if (rc) return rc;
  *bytes = layout(&tmp, nullptr);
  return SPEC_OK;
}

int spec_init(const spec_config* cfg, void* workspace, size_t ws_bytes, void* stream, spec_ctx** out) {
  if (!out) return fail(nullptr, SPEC_E_INVAL, "null out");
  *out = nullptr;
  spec_ctx* c = new (std::nothrow) spec_ctx();
  if (!c) return fail(nullptr, SPEC_E_INVAL, "host allocation failed");
  int rc = check_config(c, cfg);
  if (rc) {
    delete c;
    return rc;
  }
  rc = validate_model(c->cfg.target, "target", std::max(c->cfg.max_k, 1), c->cfg.max_batch, true);
  if (!rc && c->draft.present) rc = validate_model(c->cfg.draft, "draft", 1, c->cfg.max_batch, true);
  if (!rc && c->mtp.present) {
    const spec_mtp_desc& w = c->cfg.mtp;
    const spec_layer_weights& l = w.layer;
    if (!w.norm_h || !w.norm_e || !w.w_proj || !w.final_norm || !l.attn_norm || !l.wq || !l.wk || !l.wv ||
        !l.wo || !l.ffn_norm || !l.wg || !l.wu || !l.wd)
      rc = fail(nullptr, SPEC_E_INVAL, "mtp: null weight pointer");
  }
  if (rc) {
    delete c;
    return rc;
  }
  c->target.layers.assign(cfg->target.layers, cfg->target.layers + cfg->target.n_layers);
  c->target.d.layers = nullptr;
  if (c->target.fp8) c->target.scales.assign(cfg->target.layer_scales, cfg->target.layer_scales + cfg->target.n_layers);
  c->target.d.layer_scales = nullptr;
  if (c->draft.present) {
    c->draft.layers.assign(cfg->draft.layers, cfg->draft.layers + cfg->draft.n_layers);
    c->draft.d.layers = nullptr;
    if (c->draft.fp8) c->draft.scales.assign(cfg->draft.layer_scales, cfg->draft.layer_scales + cfg->draft.n_layers);
    c->draft.d.layer_scales = nullptr;
  }
  if (c->mtp.present) c->mtp.layers.assign(1, cfg->mtp.layer);
  const size_t need = layout(c, nullptr);
  if (!workspace || ws_bytes < need || ((uintptr_t)workspace & 255)) {
    delete c;
    return fail(nullptr, SPEC_E_INVAL, "workspace: need %zu bytes, 256-byte aligned", need);
  }
  layout(c, workspace);
  c->stream = (hipStream_t)stream;
  hipError_t e = launch_fill(workspace, need, c->stream);
  if (e == hipSuccess) e = attention_set_lds_limit();
  if (e == hipSuccess)
    e = launch_rope_table(c->target.rope, c->cap, c->target.d.head_dim, c->target.d.rope_theta, c->stream);
  if (e == hipSuccess && c->draft.present)
    e = launch_rope_table(c->draft.rope, c->cap, c->draft.d.head_dim, c->draft.d.rope_theta, c->stream);
  if (e == hipSuccess && c->mtp.present)
    e = launch_rope_table(c->mtp.rope, c->cap, c->mtp.d.head_dim, c->mtp.d.rope_theta, c->stream);
  if (e == hipSuccess) e = stream_init();
  if (e == hipSuccess) e = forward_init(&c->fgrid);
  // device copies of the layer tables (the one-launch forward reads them)
  for (Model* m : {&c->target, &c->draft}) {
    if (e != hipSuccess || !m->present) continue;
    e = hipMemcpyAsync(m->dev_layers, m->layers.data(), m->layers.size() * sizeof(spec_layer_weights),
                       hipMemcpyHostToDevice, c->stream);
  }
  if (e == hipSuccess) {
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&c->ncu, hipDeviceAttributeMultiprocessorCount, dev);
  }
  if (e != hipSuccess) {
    delete c;
    return fail(nullptr, SPEC_E_HIP, "init kernels: %s", hipGetErrorString(e));
  }
  for (Model* m : {&c->target, &c->draft}) {
    if (!m->present || !m->fp8 || stream_shapes(c, *m, m->Mmax)) continue;
    const char* name = m == &c->target ? "target" : "draft";
    delete c;
    return fail(nullptr, SPEC_E_UNSUPPORTED,
                "%s: fp8 weights need d_model in {2048, 4096}, other reductions in whole 2 KB stages", name);
  }
  *out = c;
  return SPEC_OK;
}

int spec_destroy(spec_ctx* ctx) {
  delete ctx;
  return SPEC_OK;
}

const char* spec_last_error(const spec_ctx* ctx) {
  return ctx ? ctx->err.c_str() : g_init_error.c_str();
}

int spec_load_kv(spec_ctx* c, int32_t which, int32_t seq, const void* k, const void* v, int32_t length) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (!k || !v) return fail(c, SPEC_E_INVAL, "null k / v");
  if (seq < 0 || seq >= c->cfg.max_batch) return fail(c, SPEC_E_RANGE, "seq %d", seq);
  if (length < 0 || length > c->cfg.max_ctx) return fail(c, SPEC_E_RANGE, "length %d > max_ctx", length);
  Model* m = which == 0 ? &c->target
                        : (which == 1 && c->draft.present ? &c->draft : (which == 2 && c->mtp.present ? &c->mtp : nullptr));
  if (!m) return fail(c, SPEC_E_INVAL, "cache %d not present", which);
  if (c->phase != IDLE && c->phase != READY) return fail(c, SPEC_E_STATE, "load_kv inside a cycle");
  HIPCHK(c, launch_kv_load(m->d.dtype, k, v, m->cache, seq, length, c->stream));
  if (which == 0) {
    HIPCHK(c, launch_set_len(c->len, seq, length, c->stream));
    if (!c->started) {
      c->len_lo = c->len_hi = length;
      c->started = true;
    } else {
      c->len_lo = std::min(c->len_lo, length);
      c->len_hi = std::max(c->len_hi, length);
    }
  }
  return SPEC_OK;
}

int spec_load_history(spec_ctx* c, int32_t seq, const int32_t* tokens, int32_t length) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (!tokens && length > 0) return fail(c, SPEC_E_INVAL, "null tokens");
  if (seq < 0 || seq >= c->cfg.max_batch) return fail(c, SPEC_E_RANGE, "seq %d", seq);
  if (length < 0 || length > c->cfg.max_ctx) return fail(c, SPEC_E_RANGE, "length %d > max_ctx", length);
  if (c->phase != IDLE && c->phase != READY) return fail(c, SPEC_E_STATE, "load_history inside a cycle");
  HIPCHK(c, launch_hist_write(c->hist + (int64_t)seq * c->hist_ld, c->hist_ld, tokens, length, 1, length, 0,
                              c->stream));
  return SPEC_OK;
}

int spec_set_last(spec_ctx* c, const int32_t* last_tok, const int32_t* prev_tok, const float* hidden,
                  int32_t batch) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (c->mtp.present && !hidden) return fail(c, SPEC_E_INVAL, "the MTP drafter needs the hidden state at L-1");
  if (!last_tok) return fail(c, SPEC_E_INVAL, "null last_tok");
  if (batch < 1 || batch > c->cfg.max_batch) return fail(c, SPEC_E_RANGE, "batch %d", batch);
  if (c->draft.present && !prev_tok) return fail(c, SPEC_E_INVAL, "a draft model needs prev_tok");
  if (c->phase != IDLE && c->phase != READY) return fail(c, SPEC_E_STATE, "set_last inside a cycle");
  if (!c->started) return fail(c, SPEC_E_STATE, "set_last needs a loaded cache prefix");
  HIPCHK(c, launch_copy_rows(last_tok, 1, c->last_tok, batch, c->stream));
  if (prev_tok) HIPCHK(c, launch_copy_rows(prev_tok, 1, c->prev_tok, batch, c->stream));
  HIPCHK(c, launch_hist_set_last(c->hist, c->hist_ld, c->len, last_tok, prev_tok, batch, c->stream));
  if (c->mtp.present) {
    // the head's cache prefix covers positions 0..L-1; its first row is position L
    const int d = c->mtp.d.d_model;
    HIPCHK(c, launch_copy_rows_f32(hidden, d, 1, d, batch, c->mtp_h, (int64_t)(c->cfg.max_k + 1) * d, c->stream));
    HIPCHK(c, launch_len_from(c->mtp_len, c->len, batch, 0, c->stream));
    c->mtp_rows = 1;
  }
  c->ngram_cycle = false;
  c->ctl_cycle = false;
  c->phase = READY;
  return SPEC_OK;
}

int spec_prefill(spec_ctx* c, const int32_t* tokens, int32_t batch, int32_t P) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (!tokens) return fail(c, SPEC_E_INVAL, "null tokens");
  if (batch < 1 || batch > c->cfg.max_batch) return fail(c, SPEC_E_RANGE, "batch %d", batch);
  if (P < 1) return fail(c, SPEC_E_INVAL, "P < 1");
  if (c->started && c->len_lo != c->len_hi)
    return fail(c, SPEC_E_STATE, "prefill needs equal sequence lengths");
  if (c->phase != IDLE && c->phase != READY) return fail(c, SPEC_E_STATE, "prefill inside a cycle");
  const int L0 = c->started ? c->len_hi : 0;
  if (L0 + P - 1 > c->cfg.max_ctx) return fail(c, SPEC_E_RANGE, "prompt longer than max_ctx");
  if (c->mtp.present && (L0 != 0 || P < 2))
    return fail(c, SPEC_E_UNSUPPORTED, "MTP prefill runs from an empty context over at least two tokens");
  HIPCHK(c, launch_hist_write(c->hist, c->hist_ld, tokens, P, batch, P, L0, c->stream));
  // the head's cache starts at position 1: position 0 has no previous hidden state
  if (c->mtp.present) HIPCHK(c, launch_len_from(c->mtp_len, c->len, batch, 1, c->stream));
  const int d = c->target.d.d_model;
  int done = 0, last_chunk = 0;
  while (done < P - 1) {
    const int chunk = std::min(std::min(c->target.mseq_max, P - 1 - done),
                               c->draft.present ? c->draft.mseq_max : 1 << 30);
    int rc = forward(c, c->target, batch, chunk, tokens + done, P, tokens + done + 1, P, 0, nullptr);
    if (rc) return rc;
    if (c->draft.present) {
      rc = forward(c, c->draft, batch, chunk, tokens + done, P, tokens + done + 1, P, 0, nullptr);
      if (rc) return rc;
    }
    if (c->mtp.present) {
      // head rows at positions done+1 .. from the target hidden states at done .., except
      // position P-1 (the last token's), which the first draft_step computes
      const int cnt = (done + chunk == P - 1) ? chunk - 1 : chunk;
      if (cnt > 0) {
        rc = mtp_layer(c, batch, cnt, c->target.x, (int64_t)chunk * d, tokens + done + 1, P, nullptr, 0);
        if (rc) return rc;
        HIPCHK(c, launch_add_len(c->mtp_len, batch, cnt, c->stream));
      }
    }
    HIPCHK(c, launch_add_len(c->len, batch, chunk, c->stream));
    done += chunk;
    last_chunk = chunk;
  }
  if (c->mtp.present) {
    HIPCHK(c, launch_copy_rows_f32(c->target.x + (int64_t)(last_chunk - 1) * d, (int64_t)last_chunk * d, 1, d,
                                   batch, c->mtp_h, (int64_t)(c->cfg.max_k + 1) * d, c->stream));
    c->mtp_rows = 1;
  }
  HIPCHK(c, launch_copy_rows(tokens + (P - 1), P, c->last_tok, batch, c->stream));
  if (P >= 2) HIPCHK(c, launch_copy_rows(tokens + (P - 2), P, c->prev_tok, batch, c->stream));
  c->ngram_cycle = false;
  c->ctl_cycle = false;
  c->len_lo = c->len_hi = L0 + P - 1;
  c->started = true;
  c->phase = READY;
  return SPEC_OK;
}

int draft_step(spec_ctx* c, int32_t batch, int32_t k, uint64_t round, int32_t* draft_tok, spec_probs* q,
               int32_t* n_drafted) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (int rc = cycle_usable(c)) return rc;
  const int kind = c->cfg.draft_kind;
  if (kind == SPEC_DRAFT_NONE) return fail(c, SPEC_E_UNSUPPORTED, "no drafter configured");
  if (batch < 1 || batch > c->cfg.max_batch) return fail(c, SPEC_E_RANGE, "batch %d", batch);
  if (k < 1 || k > c->cfg.max_k) return fail(c, SPEC_E_RANGE, "k %d not in 1..max_k", k);
  if (!draft_tok) return fail(c, SPEC_E_INVAL, "null draft_tok");
  int rc = check_probs(c, q, "q", list_cap(c->cfg.sampler));
  if (rc) return rc;
  if (c->phase != READY) return fail(c, SPEC_E_STATE, "draft_step needs a start (prefill / set_last) or a trimmed cycle");
  if (kind == SPEC_DRAFT_MODEL && c->len_lo < 1)
    return fail(c, SPEC_E_STATE, "draft model needs a token before the last one");
  // the MTP catch-up writes its cache up to mtp_rows - 1 positions past L
  rc = ensure_room(c, batch, std::max(k, kind == SPEC_DRAFT_MTP ? c->mtp_rows : 0) + 1);
  if (rc) return rc;
  const NchScope nch(c, std::max(k, kind == SPEC_DRAFT_MTP ? c->mtp_rows : 0) + 1);
  const spec_probs qq = *q;
  c->ctl_cycle = c->p_min > 0.0f || c->min_draft > 0;
  if (kind == SPEC_DRAFT_NGRAM) {
    rc = enqueue_draft_ngram(c, batch, k, draft_tok, qq);
    if (rc) return rc;
    std::vector<int32_t> found(batch);
    HIPCHK(c, hipMemcpyAsync(found.data(), c->ndraft, sizeof(int32_t) * batch, hipMemcpyDeviceToHost, c->stream));
    HIPCHK(c, hipStreamSynchronize(c->stream));
    int mx = 0;
    for (int b = 0; b < batch; ++b) mx = std::max(mx, found[b]);
    if (n_drafted) *n_drafted = mx;
    c->ngram_cycle = true;
  } else {
    if (c->p_min > 0.0f && batch > 64) return fail(c, SPEC_E_UNSUPPORTED, "draft probability with more than 64 sequences");
    HIPCHK(c, launch_set_u32(c->round_dev, (uint32_t)round, c->stream));
    uint32_t pbits = 0;
    std::memcpy(&pbits, &c->p_min, sizeof pbits);
    // the threshold is part of the captured launches (the controlled sampling kernel's argument)
    const void* key[8] = {draft_tok, qq.ids, qq.probs, qq.count, (const void*)(intptr_t)qq.cap,
                          (const void*)(intptr_t)(kind == SPEC_DRAFT_MTP ? c->mtp_rows : 0),
                          (const void*)(uintptr_t)pbits, (const void*)(intptr_t)c->attn_nch};
    if (kind == SPEC_DRAFT_MTP)
      rc = run_graphed(c, 2, batch, k, key, [&]() { return enqueue_draft_mtp(c, batch, k, draft_tok, qq); });
    else
      rc = run_graphed(c, 1, batch, k, key, [&]() { return enqueue_draft(c, batch, k, draft_tok, qq); });
    if (rc) return rc;
    if (n_drafted) *n_drafted = k;
  }
  c->phase = DRAFTED;
  c->phase_k = k;
  c->phase_batch = batch;
  return SPEC_OK;
}

int verify_step(spec_ctx* c, const int32_t* draft_tok, int32_t batch, int32_t k, float* logits_out,
                spec_probs* p) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (int rc = cycle_usable(c)) return rc;
  if (batch < 1 || batch > c->cfg.max_batch) return fail(c, SPEC_E_RANGE, "batch %d", batch);
  if (k < 0 || k > c->cfg.max_k) return fail(c, SPEC_E_RANGE, "k %d not in 0..max_k", k);
  if (k > 0 && !draft_tok) return fail(c, SPEC_E_INVAL, "null draft_tok");
  int rc = check_probs(c, p, "p", list_cap(c->cfg.sampler));
  if (rc) return rc;
  if (c->phase != READY && c->phase != DRAFTED)
    return fail(c, SPEC_E_STATE, "verify_step needs a start (prefill / set_last) or a trimmed cycle");
  if (c->mtp.present && c->phase != DRAFTED)
    return fail(c, SPEC_E_STATE, "with the MTP drafter every cycle starts with draft_step (the head catches up "
                                 "only from the previous verify)");
  if (c->phase == DRAFTED && c->ngram_cycle && batch > 1 && k != c->phase_k)
    return fail(c, SPEC_E_INVAL, "n-gram drafts of a batch are verified at the drafted k (row stride)");
  if (c->phase == DRAFTED && k > c->phase_k) return fail(c, SPEC_E_INVAL, "k > drafted k");
  if (c->phase == READY) {
    c->ngram_cycle = false;
    c->ctl_cycle = false;
  }
  rc = ensure_room(c, batch, k + 1);
  if (rc) return rc;
  const NchScope nch(c, k + 1);
  const spec_probs pp = *p;
  const void* key[8] = {draft_tok, logits_out, pp.ids, pp.probs, pp.count, (const void*)(intptr_t)pp.cap,
                        (const void*)(intptr_t)c->attn_nch, nullptr};
  rc = run_graphed(c, 0, batch, k, key, [&]() { return enqueue_verify(c, draft_tok, batch, k, logits_out, pp); });
  if (rc) return rc;
  c->phase = VERIFIED;
  c->phase_k = k;
  c->phase_batch = batch;
  return SPEC_OK;
}

int accept(spec_ctx* c, const int32_t* draft_tok, const spec_probs* q, const spec_probs* p, int32_t batch,
           int32_t k, uint64_t round, int32_t* n_acc, int32_t* out_tok, uint8_t* near_tie) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (int rc = cycle_usable(c)) return rc;
  if (c->phase != VERIFIED) return fail(c, SPEC_E_STATE, "accept must follow verify_step");
  if (k != c->phase_k || batch != c->phase_batch) return fail(c, SPEC_E_STATE, "k / batch differ from the verify");
  if (!n_acc || !out_tok || (k > 0 && !draft_tok)) return fail(c, SPEC_E_INVAL, "null output");
  const int greedy = !(c->cfg.sampler.temperature > 0.0f);
  int rc = check_probs(c, p, "p", 1);
  if (rc) return rc;
  if (k > 0 && !greedy) {
    rc = check_probs(c, q, "q", 1);
    if (rc) return rc;
  }
  AcceptArgs a{};
  a.drafts = draft_tok;
  if (q) a.q = *q;
  a.p = *p;
  a.batch = batch;
  a.k = k;
  a.greedy = greedy;
  a.seed = c->cfg.seed;
  a.round = (uint32_t)round;
  a.n_acc = n_acc;
  a.out_tok = out_tok;
  a.near_tie = near_tie;
  a.last_tok = c->last_tok;
  a.prev_tok = c->prev_tok;
  a.stats = c->stats;
  // drafts proposed per sequence: the n-gram lookup's count, or the draft model's / MTP
  // head's kept count under a draft-probability threshold; then the minimum worth checking
  const bool kept = c->ctl_cycle && c->p_min > 0.0f && c->cfg.draft_kind != SPEC_DRAFT_NGRAM;
  a.kcap = (c->ngram_cycle || kept) ? c->ndraft : nullptr;
  a.min_draft = c->ctl_cycle ? c->min_draft : 0;
  a.hist = c->hist;
  a.hist_ld = c->hist_ld;
  a.len = c->len;
  LAUNCH(c, PROF_ACCEPT, launch_accept(a, c->stream));
  c->phase = ACCEPTED;
  return SPEC_OK;
}

int kv_trim(spec_ctx* c, const int32_t* n_acc, int32_t batch) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (int rc = cycle_usable(c)) return rc;
  if (c->phase != ACCEPTED) return fail(c, SPEC_E_STATE, "kv_trim must follow accept");
  if (batch != c->phase_batch) return fail(c, SPEC_E_STATE, "batch differs from the cycle");
  if (!n_acc) return fail(c, SPEC_E_INVAL, "null n_acc");
  LAUNCH(c, PROF_TRIM, launch_trim(c->len, n_acc, batch, c->phase_k, c->mtp.present ? c->mtp_len : nullptr, c->stream));
  c->len_lo += 1;
  c->len_hi += 1 + c->phase_k;
  c->mtp_rows = c->phase_k + 1;
  c->ngram_cycle = false;
  c->ctl_cycle = false;
  c->phase = READY;
  return SPEC_OK;
}

int spec_draft_controls(spec_ctx* c, float p_min, int32_t min_draft) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (!(p_min >= 0.0f && p_min <= 1.0f)) return fail(c, SPEC_E_INVAL, "draft probability %g not in [0, 1]", p_min);
  if (min_draft < 0) return fail(c, SPEC_E_INVAL, "min_draft < 0");
  if (c->phase != IDLE && c->phase != READY) return fail(c, SPEC_E_STATE, "draft controls change between cycles");
  c->p_min = p_min;
  c->min_draft = min_draft;
  return SPEC_OK;
}

int spec_profile(spec_ctx* c, int32_t enable) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  c->prof = enable != 0;
  return SPEC_OK;
}

int spec_profile_repeat(spec_ctx* c, int32_t slot, int32_t reps) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (reps < 1 || reps > 64) return fail(c, SPEC_E_INVAL, "reps must be 1..64");
  if (slot < 0 || slot >= SPEC_PROF_SLOTS || slot % 16 != PROF_GATEUP)
    return fail(c, SPEC_E_INVAL, "only the gate/up slots can repeat");
  c->prof_rep_slot = reps > 1 ? slot : -1;
  c->prof_reps = reps;
  return SPEC_OK;
}

int spec_profile_read(spec_ctx* c, double* ms, int64_t* launches) {
  if (need_ctx(c) || !ms || !launches) return SPEC_E_INVAL;
  HIPCHK(c, hipStreamSynchronize(c->stream));
  for (int i = 0; i < SPEC_PROF_SLOTS; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  for (auto& r : c->recs) {
    float t = 0.0f;
    HIPCHK(c, hipEventElapsedTime(&t, r.a, r.b));
    ms[r.slot] += t;
    launches[r.slot] += r.reps;
    c->ev_free.push_back(r.a);
    c->ev_free.push_back(r.b);
  }
  c->recs.clear();
  return SPEC_OK;
}

int spec_use_gemv(spec_ctx* c, int32_t enable) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  c->draft.gemv = enable != 0 && c->draft.present;
  return SPEC_OK;
}

int spec_set_schedule(spec_ctx* c, int32_t schedule) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (schedule != SPEC_SCHED_STEP && schedule != SPEC_SCHED_STREAM && schedule != SPEC_SCHED_FORWARD)
    return fail(c, SPEC_E_INVAL, "schedule %d", schedule);
  c->sched = schedule;
  return SPEC_OK;
}

int spec_trace_forward(spec_ctx* c, void* buf, int64_t bytes, int32_t* grid) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (grid) *grid = c->fgrid;
  if (!buf || c->fgrid < 1) {
    c->ftrace = nullptr;
    c->ftrace_cap = 0;
    return SPEC_OK;
  }
  const int64_t per = (int64_t)c->fgrid * 2 * 8;
  if (bytes < per) return fail(c, SPEC_E_INVAL, "trace buffer: need at least %lld bytes", (long long)per);
  c->ftrace = (unsigned long long*)buf;
  c->ftrace_cap = (int)std::min<int64_t>(bytes / per, 1 << 20);
  return SPEC_OK;
}

int spec_use_graphs(spec_ctx* c, int32_t enable) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  c->graphs = enable != 0;
  return SPEC_OK;
}

int spec_get_stats(spec_ctx* c, spec_stats* out) {
  if (need_ctx(c) || !out) return SPEC_E_INVAL;
  int64_t h[4];
  HIPCHK(c, hipMemcpyAsync(h, c->stats, sizeof h, hipMemcpyDeviceToHost, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  out->cycles = h[0];
  out->drafts_attempted = h[1];
  out->drafts_accepted = h[2];
  out->emitted = h[3];
  unsigned err = 0;
  HIPCHK(c, hipMemcpyAsync(&err, (const char*)c->fsync + forward_error_offset(), sizeof err,
                           hipMemcpyDeviceToHost, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  out->sync_timeouts = err;
  if (err) {
    c->barrier_failed = true;
    return fail(c, SPEC_E_HIP, "a grid barrier of the one-launch forward timed out");
  }
  return SPEC_OK;
}

int spec_get_lengths(spec_ctx* c, int32_t* lengths, int32_t batch) {
  if (need_ctx(c) || !lengths) return SPEC_E_INVAL;
  if (batch < 1 || batch > c->cfg.max_batch) return fail(c, SPEC_E_RANGE, "batch %d", batch);
  HIPCHK(c, hipMemcpyAsync(lengths, c->len, sizeof(int32_t) * batch, hipMemcpyDeviceToHost, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  return read_barrier_error(c);
}

int spec_debug_read(spec_ctx* c, int32_t which, int32_t buffer, void* dst, size_t bytes) {
  if (need_ctx(c) || !dst) return SPEC_E_INVAL;
  Model* m = which == 0 ? &c->target : (which == 1 ? &c->draft : (which == 2 ? &c->mtp : nullptr));
  if (!m || !m->present) return fail(c, SPEC_E_INVAL, "no model %d", which);
  const spec_model_desc& d = m->d;
  const size_t rows = (size_t)m->Mmax;
  const size_t cache = (size_t)c->cfg.max_batch * d.n_layers * d.n_kv_heads * c->cap * d.head_dim * m->act;
  const void* src = nullptr;
  size_t n = 0;
  switch (buffer) {
    case SPEC_BUF_RESIDUAL: src = m->x; n = rows * d.d_model * 4; break;
    case SPEC_BUF_NORM_INPUT: src = m->xn; n = rows * d.d_model * 4; break;
    case SPEC_BUF_Q: src = m->qst; n = rows * m->q_dim * 4; break;
    case SPEC_BUF_K: src = m->kst; n = rows * m->kv_dim * 4; break;
    case SPEC_BUF_ATTN: src = m->attn; n = rows * m->q_dim * m->act; break;
    case SPEC_BUF_SWIGLU: src = m->h; n = rows * d.d_ffn * m->act; break;
    case SPEC_BUF_CACHE_K: src = m->cache.k; n = cache; break;
    case SPEC_BUF_CACHE_V: src = m->cache.v; n = cache; break;
    case SPEC_BUF_LOGITS: src = m->logits; n = (size_t)m->logit_rows * d.vocab * 4; break;
    default: return fail(c, SPEC_E_INVAL, "unknown buffer %d", buffer);
  }
  if (bytes < n) n = bytes;
  HIPCHK(c, hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, c->stream));
  return SPEC_OK;
}

// ---------------------------------------------------------------- n-gram gate (host)
int spec_gate_init(spec_gate* g, int32_t n_max, const double* verify_cost, double draft_cost, int32_t enabled) {
  if (!g || !verify_cost || n_max < 0 || n_max > SPEC_MAX_K) return SPEC_E_INVAL;
  if (!(verify_cost[0] > 0.0) || !(draft_cost >= 0.0)) return SPEC_E_INVAL;
  for (int k = 0; k <= n_max; ++k)
    if (!(verify_cost[k] > 0.0)) return SPEC_E_INVAL;
  g->n_max = n_max;
  g->enabled = enabled != 0;
  g->weight = 0.5;
  g->alpha = 1.0;
  for (int k = 0; k <= SPEC_MAX_K; ++k) g->cost[k] = k <= n_max ? verify_cost[k] / verify_cost[0] : 0.0;
  g->draft_cost = draft_cost / verify_cost[0];
  return SPEC_OK;
}

int32_t spec_gate_choose(const spec_gate* g) {
  if (!g) return SPEC_E_INVAL;
  if (!g->enabled) return g->n_max;
  int best_k = 0;
  double best_v = -1.0;
  for (int k = 0; k <= g->n_max; ++k) {
    // expected tokens of a step that drafts k (1 + alpha + ... + alpha^k) over its cost
    double gain = 0.0;
    for (int i = 0; i <= k; ++i) gain += std::pow(g->alpha, (double)i);
    const double v = gain / (g->cost[k] + k * g->draft_cost);
    if (v > best_v + 1e-12) {
      best_k = k;
      best_v = v;
    }
  }
  return best_k;
}

int spec_gate_update(spec_gate* g, int32_t accepted, int32_t attempted) {
  if (!g || accepted < 0 || attempted < 0 || accepted > attempted) return SPEC_E_INVAL;
  if (attempted > 0) g->alpha = g->weight * g->alpha + (1.0 - g->weight) * ((double)accepted / (double)attempted);
  return SPEC_OK;
}

// ---------------------------------------------------------------- adaptive depth (host)
int spec_depth_init(spec_depth* d, int32_t k0, int32_t k_min, int32_t k_max, int32_t up, int32_t down) {
  if (!d || k_min < 0 || k0 < k_min || k_max < k0 || k_max > SPEC_MAX_K || up < 0 || down < 0) return SPEC_E_INVAL;
  d->k = k0;
  d->k_min = k_min;
  d->k_max = k_max;
  d->up = up;
  d->down = down;
  return SPEC_OK;
}

int32_t spec_depth_choose(const spec_depth* d) { return d ? d->k : SPEC_E_INVAL; }

int spec_depth_update(spec_depth* d, int32_t accepted, int32_t attempted) {
  if (!d || accepted < 0 || accepted > attempted) return SPEC_E_INVAL;
  if (attempted == 0) return SPEC_OK;
  d->k = accepted == attempted ? std::min(d->k_max, d->k + d->up) : std::max(d->k_min, d->k - d->down);
  return SPEC_OK;
}

// ---------------------------------------------------------------- stateless
int spec_truncate_scratch_size(int32_t rows, int32_t vocab, size_t* bytes) {
  if (!bytes || rows < 0 || vocab < 1) return SPEC_E_INVAL;
  return truncate_scratch_bytes(rows, vocab, bytes);
}

int spec_truncate(const void* logits, int32_t dtype, int32_t rows, int32_t vocab, int64_t row_stride,
                  const spec_sampler* s, spec_probs* out, uint8_t* flags, void* scratch, size_t scratch_bytes,
                  void* stream) {
  if (!logits || !s || !out || !scratch || rows < 0 || vocab < 1 || row_stride < vocab) return SPEC_E_INVAL;
  if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16) return SPEC_E_INVAL;
  int rc = validate_sampler(*s);
  if (rc) return rc;
  if (s->temperature > 0.0f && s->top_k > vocab) return SPEC_E_INVAL;
  if (!out->ids || !out->probs || !out->count || out->cap < list_cap(*s)) return SPEC_E_INVAL;
  size_t need = 0;
  rc = truncate_scratch_bytes(rows, vocab, &need);
  if (rc) return rc;
  if (scratch_bytes < need) return SPEC_E_RANGE;
  return launch_truncate(logits, dtype, rows, vocab, row_stride, *s, *out, 1, flags, scratch,
                         (hipStream_t)stream) == hipSuccess ? SPEC_OK : SPEC_E_HIP;
}

// ---------------------------------------------------------------- truncation without allocation
// The truncation's partial lists and flags live in this fixed device array instead of a caller
// workspace.  Each device holds its own copy at its own address: host code never passes the
// array's name to a kernel (on the host it names a stand-in, not device memory) but the
// address hipGetSymbolAddress returns, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

static constexpr int NOALLOC_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

// The current device's copy of `scratch`, looked up on the first call on that device.
static int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SPEC_E_HIP;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return SPEC_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return SPEC_E_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SPEC_OK;
}

int spec_truncate_noalloc(const void* logits, int32_t dtype, int32_t rows, int32_t vocab,
                          int64_t row_stride, const spec_sampler* s, spec_probs* out, uint8_t* flags,
                          void* stream) {
  if (!logits || !s || !out || rows < 0 || vocab < 1 || row_stride < vocab) return SPEC_E_INVAL;
  if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16) return SPEC_E_INVAL;
  int rc = validate_sampler(*s);
  if (rc) return rc;
  if (s->temperature > 0.0f && s->top_k > vocab) return SPEC_E_INVAL;
  if (!out->ids || !out->probs || !out->count || out->cap < list_cap(*s)) return SPEC_E_INVAL;
  size_t need = 0;
  rc = truncate_scratch_bytes(rows, vocab, &need);
  if (rc) return rc;
  if (need > (size_t)SPEC_NOALLOC_SCRATCH_BYTES) return SPEC_E_RANGE;
  void* ptr = nullptr;
  rc = noalloc_scratch(&ptr);
  if (rc) return rc;
  // every slot the kernels read is written first in the same call: nothing to clear
  return launch_truncate(logits, dtype, rows, vocab, row_stride, *s, *out, 1, flags, ptr,
                         (hipStream_t)stream) == hipSuccess ? SPEC_OK : SPEC_E_HIP;
}

int spec_sample(const spec_probs* lists, int32_t batch, int32_t per_seq, uint64_t seed, uint64_t round,
                int32_t stream_id, int32_t* tokens, uint8_t* flags, void* stream) {
  if (!lists || !lists->ids || !lists->probs || !lists->count || !tokens) return SPEC_E_INVAL;
  if (batch < 0 || per_seq < 1 || lists->cap < 1 || stream_id < 0) return SPEC_E_INVAL;
  return launch_sample(*lists, 1, batch * per_seq, per_seq, 1, seed, nullptr, (uint32_t)round,
                       (uint32_t)stream_id, tokens, per_seq, flags, (hipStream_t)stream) == hipSuccess
             ? SPEC_OK
             : SPEC_E_HIP;
}

int spec_accept_lists(const int32_t* draft_tok, const spec_probs* q, const spec_probs* p, int32_t batch,
                      int32_t k, int32_t greedy, uint64_t seed, uint64_t round, int32_t* n_acc,
                      int32_t* out_tok, uint8_t* near_tie, void* stream) {
  if (!p || !p->ids || !p->probs || !p->count || !n_acc || !out_tok) return SPEC_E_INVAL;
  if (batch < 0 || k < 0 || k > SPEC_MAX_K) return SPEC_E_INVAL;
  if (k > 0 && (!draft_tok || (!greedy && (!q || !q->ids || !q->probs || !q->count)))) return SPEC_E_INVAL;
  if (p->cap > SPEC_TOPK_MAX || (q && q->cap > SPEC_TOPK_MAX)) return SPEC_E_UNSUPPORTED;
  AcceptArgs a{};
  a.drafts = draft_tok;
  if (q) a.q = *q;
  a.p = *p;
  a.batch = batch;
  a.k = k;
  a.greedy = greedy ? 1 : 0;
  a.seed = seed;
  a.round = (uint32_t)round;
  a.n_acc = n_acc;
  a.out_tok = out_tok;
  a.near_tie = near_tie;
  return launch_accept(a, (hipStream_t)stream) == hipSuccess ? SPEC_OK : SPEC_E_HIP;
}

static_assert(GDN_MAX_TOKENS == SPEC_GDN_MAX_TOKENS && GDN_DK == 128, "gdn limits");

int spec_gdn_commit_forward(const spec_gdn_shape* shape, float* state, const float* q, const float* k,
                            const float* v, const float* alpha, const float* beta, int32_t n_commit,
                            int32_t n_fwd, float* out, void* stream) {
  if (!shape) return fail(nullptr, SPEC_E_INVAL, "gdn: null shape");
  if (shape->n_heads < 1 || shape->d_v < 1 || shape->d_k < 1 || n_commit < 0 || n_fwd < 0)
    return fail(nullptr, SPEC_E_INVAL, "gdn: non-positive shape or negative token count");
  if (shape->d_k != GDN_DK || shape->d_v % 32)
    return fail(nullptr, SPEC_E_UNSUPPORTED, "gdn: d_k must be %d and d_v a multiple of 32", GDN_DK);
  if (n_commit > GDN_MAX_TOKENS || n_fwd > GDN_MAX_TOKENS || n_commit + n_fwd > GDN_MAX_TOKENS)
    return fail(nullptr, SPEC_E_RANGE, "gdn: more than %d tokens in one call", GDN_MAX_TOKENS);
  if (n_commit + n_fwd == 0) return SPEC_OK;
  if (!state || !k || !v || !alpha || !beta || (n_fwd > 0 && (!q || !out)))
    return fail(nullptr, SPEC_E_INVAL, "gdn: null pointer");
  // the kernel's LDS limit is a per-device attribute: set it once on each device used
  static std::atomic<bool> ready[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(nullptr, SPEC_E_HIP, "gdn: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(nullptr, SPEC_E_UNSUPPORTED, "gdn: device %d", dev);
  if (!ready[dev].load()) {
    e = gdn_init();
    if (e != hipSuccess) return fail(nullptr, SPEC_E_HIP, "gdn init: %s", hipGetErrorString(e));
    ready[dev].store(true);
  }
  GdnArgs a{};
  a.state = state;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  a.n_heads = shape->n_heads;
  a.d_v = shape->d_v;
  a.n_commit = n_commit;
  a.n_fwd = n_fwd;
  e = launch_gdn(a, (hipStream_t)stream);
  return e == hipSuccess ? SPEC_OK : fail(nullptr, SPEC_E_HIP, "gdn launch: %s", hipGetErrorString(e));
}

int spec_philox_uniforms(uint64_t seed, const uint32_t* ctr, int32_t n, float* out, void* stream) {
  if (!ctr || !out || n < 0) return SPEC_E_INVAL;
  return launch_philox(seed, ctr, n, out, (hipStream_t)stream) == hipSuccess ? SPEC_OK : SPEC_E_HIP;
}

int spec_ngram_match(const int32_t* ctx, const int32_t* lengths, int32_t batch, int32_t ld, int32_t k,
                     int32_t n_min, int32_t max_match, int32_t* drafts, int32_t* n_found, int32_t* match,
                     void* stream) {
  if (!ctx || !lengths || !drafts || !n_found || !match) return SPEC_E_INVAL;
  if (batch < 0 || ld < 1 || k < 1 || n_min < 1 || max_match < n_min) return SPEC_E_INVAL;
  NgramArgs a{ctx, lengths, batch, ld, k, n_min, max_match, 0, drafts, n_found, match};
  return launch_ngram(a, (hipStream_t)stream) == hipSuccess ? SPEC_OK : SPEC_E_HIP;
}

}  // extern "C"
