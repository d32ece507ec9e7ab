// Host side of the C ABI: validation, workspace carving, the forward sequence of each
// model, and the draft / verify / accept / trim state machine.  No device allocation.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
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

struct Model {
  int mi = 0;  // 0 target, 1 draft (profiling slot offset 16 * mi)
  spec_model_desc d{};
  std::vector<spec_layer_weights> layers;
  bool present = false;
  int q_dim = 0, kv_dim = 0, mseq_max = 0, Mmax = 0, nchunk = 0;
  size_t act = 4;
  CacheView cache{};
  float* x = nullptr;
  void* xn = nullptr;
  float* qst = nullptr;
  float* kst = nullptr;
  void* attn = nullptr;
  void* h = nullptr;
  float* logits = nullptr;
  float* part = nullptr;
  float* ss = nullptr;  // [Mmax][d/16] partial sums of squares of the residual rows
  float2* rope = nullptr;
};

// IDLE: nothing to decode from yet; READY: a last token is set, the caches are trimmed;
// DRAFTED / VERIFIED / ACCEPTED: inside a cycle.
enum Phase { IDLE = 0, READY = 1, DRAFTED = 2, VERIFIED = 3, ACCEPTED = 4 };

enum ProfClass {
  PROF_EMBED = 0, PROF_NORM = 1, PROF_QKV = 2, PROF_ATTN = 3, PROF_OPROJ = 4, PROF_GATEUP = 5,
  PROF_DOWN = 6, PROF_LMHEAD = 7, PROF_TRUNC = 8, PROF_SAMPLE = 9, PROF_ACCEPT = 10, PROF_TRIM = 11
};

struct ProfRec {
  int slot;
  hipEvent_t a, b;
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
  Model target, draft;
  hipStream_t stream = nullptr;
  int32_t* len = nullptr;       // [max_batch] context length L per sequence
  int32_t* last_tok = nullptr;  // [max_batch] token at position L
  int32_t* prev_tok = nullptr;  // [max_batch] token at position L-1
  int64_t* stats = nullptr;     // 4 counters
  void* trunc = nullptr;
  size_t trunc_bytes = 0;
  int cap = 0;
  // host bookkeeping: every sequence's L lies in [len_lo, len_hi]
  int len_lo = 0, len_hi = 0;
  bool started = false;
  Phase phase = IDLE;
  int phase_k = -1, phase_batch = -1;
  uint32_t* round_dev = nullptr;  // the cycle's round, read by the draft sampling kernels
  // launch profiling (events around every launch; graphs are bypassed while it is on)
  bool prof = false;
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
      (ctx)->recs.push_back(ProfRec{(slot), ea_, eb_});                    \
    }                                                                      \
  } while (0)

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

int validate_model(const spec_model_desc& m, const char* name, int max_k, int max_batch, bool need_w) {
  if (m.n_layers < 1 || m.d_model < 16 || m.n_q_heads < 1 || m.n_kv_heads < 1 || m.head_dim < 2 ||
      m.d_ffn < 16 || m.vocab < 2)
    return fail(nullptr, SPEC_E_INVAL, "%s: non-positive shape", name);
  if (m.dtype != SPEC_DTYPE_F32 && m.dtype != SPEC_DTYPE_BF16)
    return fail(nullptr, SPEC_E_INVAL, "%s: dtype %d", name, m.dtype);
  if (m.head_dim != 32 && m.head_dim != 64 && m.head_dim != 128)
    return fail(nullptr, SPEC_E_UNSUPPORTED, "%s: head_dim %d (32, 64 or 128)", name, m.head_dim);
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
  const int rmax = m.dtype == SPEC_DTYPE_BF16 ? GEMM_MAX_ROWS_BF16 : GEMM_MAX_ROWS_F32;
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
  const int rmax = m.dtype == SPEC_DTYPE_BF16 ? GEMM_MAX_ROWS_BF16 : GEMM_MAX_ROWS_F32;
  int r = std::max(max_k + 1, PREFILL_ROWS);
  r = std::min(r, ATTN_ROWS_MAX / G);
  r = std::min(r, rmax / max_batch);
  return std::max(r, max_k + 1);
}

void carve_model(Model& m, Carver& cv, int B, int cap) {
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
  m.xn = cv.take<void>((size_t)m.Mmax * d.d_model * m.act);
  m.qst = cv.take<float>((size_t)m.Mmax * m.q_dim * 4);
  m.kst = cv.take<float>((size_t)m.Mmax * m.kv_dim * 4);
  m.attn = cv.take<void>((size_t)m.Mmax * m.q_dim * m.act);
  m.h = cv.take<void>((size_t)m.Mmax * d.d_ffn * m.act);
  m.logits = cv.take<float>((size_t)m.Mmax * d.vocab * 4);
  m.part = cv.take<float>((size_t)m.Mmax * d.n_q_heads * m.nchunk * (d.head_dim + 2) * 4);
  m.ss = cv.take<float>((size_t)m.Mmax * (d.d_model / 16 + 1) * 4);
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
  c->target.mseq_max = max_rows_per_seq(c->target.d, g.max_k, B);
  carve_model(c->target, cv, B, c->cap);
  if (c->draft.present) {
    c->draft.mseq_max = std::max(2, max_rows_per_seq(c->draft.d, 1, B));
    carve_model(c->draft, cv, B, c->cap);
  }
  size_t tb = 0;
  const int rows = std::max(c->target.Mmax, c->draft.present ? c->draft.Mmax : 0);
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
  c->target.d = g.target;
  c->target.present = true;
  c->target.mi = 0;
  if (g.draft_kind == SPEC_DRAFT_MODEL) {
    rc = validate_model(g.draft, "draft", 1, g.max_batch, false);
    if (rc) return rc;
    if (g.draft.vocab != g.target.vocab)
      return fail(nullptr, SPEC_E_INVAL, "draft vocab %d != target vocab %d", g.draft.vocab, g.target.vocab);
    c->draft.d = g.draft;
    c->draft.present = true;
    c->draft.mi = 1;
  } else if (g.draft_kind != SPEC_DRAFT_NONE) {
    return fail(nullptr, SPEC_E_UNSUPPORTED, "draft kind %d is not implemented by this library build",
                g.draft_kind);
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

// One forward of model m over M = B*mseq rows; rows' tokens come from first/rest (see
// launch_embed) at positions len + pos_off + i.  Logits go to `logits` when non-null.
int forward(spec_ctx* c, Model& m, int B, int mseq, const int32_t* first, int first_ld,
            const int32_t* rest, int rest_ld, int pos_off, float* logits) {
  const spec_model_desc& d = m.d;
  const hipStream_t st = c->stream;
  const int M = B * mseq;
  const int dt = d.dtype;
  const int P = 16 * m.mi;
  // bf16 models fuse each RMSNorm into the projection that consumes it (see gemm_bf16_kernel);
  // f32 models run it as its own kernel
  const bool fused = dt == SPEC_DTYPE_BF16;
  const int ss_ld = d.d_model / 16 + 1;
  LAUNCH(c, P + PROF_EMBED, launch_embed(dt, d.embed, d.d_model, d.vocab, first, first_ld, rest, rest_ld, M, mseq,
                                         m.x, fused ? m.ss : nullptr, ss_ld, st));
  int np = 1;  // partial sums of squares per row available in m.ss
  RowMap rm{M, mseq, c->len, pos_off};
  // Few rows (the draft, plain decoding): every projection workgroup normalizes them itself
  // in its LDS prologue, which saves a launch.  More rows: one stand-alone kernel with the
  // same arithmetic writes them once (redoing them in every workgroup costs more).
  const bool in_lds = (int64_t)M * d.d_model <= 4096 && gemm_norm_lds_bytes(M, d.d_model) <= GEMM_NORM_LDS_MAX;
  auto norm_input = [&](GemmArgs& g, const void* gain) -> int {
    if (fused && in_lds) {
      g.xres = m.x;
      g.gain = gain;
      g.ss_in = m.ss;
      g.np_in = np;
      g.ss_ld = ss_ld;
      g.eps = d.rms_eps;
    } else {
      if (fused)
        LAUNCH(c, P + PROF_NORM, launch_norm_apply(m.x, gain, m.ss, np, ss_ld, d.rms_eps, M, d.d_model, m.xn, st));
      g.x = m.xn;
    }
    return SPEC_OK;
  };
  for (int l = 0; l < d.n_layers; ++l) {
    const spec_layer_weights& w = m.layers[l];
    if (!fused) LAUNCH(c, P + PROF_NORM, launch_rmsnorm(dt, m.x, w.attn_norm, d.rms_eps, M, d.d_model, m.xn, st));
    GemmArgs g{};
    g.w[0] = w.wq;
    g.w[1] = w.wk;
    g.w[2] = w.wv;
    g.rows[0] = m.q_dim;
    g.rows[1] = m.kv_dim;
    g.rows[2] = m.kv_dim;
    g.K = d.d_model;
    if (norm_input(g, w.attn_norm)) return SPEC_E_HIP;
    g.rm = rm;
    g.q_stage = m.qst;
    g.k_stage = m.kst;
    g.cache = m.cache;
    g.layer = l;
    LAUNCH(c, P + PROF_QKV, launch_gemm(dt, EPI_QKV, g, st));
    AttnArgs a{};
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
    a.out = m.attn;
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
    LAUNCH(c, P + PROF_OPROJ, launch_gemm(dt, EPI_RESID, o, st));
    np = d.d_model / 16;
    if (!fused) LAUNCH(c, P + PROF_NORM, launch_rmsnorm(dt, m.x, w.ffn_norm, d.rms_eps, M, d.d_model, m.xn, st));
    GemmArgs gu{};
    gu.w[0] = w.wg;
    gu.w[1] = w.wu;
    gu.rows[0] = d.d_ffn;
    gu.K = d.d_model;
    if (norm_input(gu, w.ffn_norm)) return SPEC_E_HIP;
    gu.rm = rm;
    gu.h = m.h;
    LAUNCH(c, P + PROF_GATEUP, launch_gemm(dt, EPI_SWIGLU, gu, st));
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
    LAUNCH(c, P + PROF_DOWN, launch_gemm(dt, EPI_RESID, dn, st));
  }
  if (logits) {
    if (!fused) LAUNCH(c, P + PROF_NORM, launch_rmsnorm(dt, m.x, d.final_norm, d.rms_eps, M, d.d_model, m.xn, st));
    GemmArgs lm{};
    lm.w[0] = d.lm_head;
    lm.rows[0] = d.vocab;
    lm.K = d.d_model;
    if (norm_input(lm, d.final_norm)) return SPEC_E_HIP;
    lm.rm = rm;
    lm.out = logits;
    lm.ld = d.vocab;
    LAUNCH(c, P + PROF_LMHEAD, launch_gemm(dt, EPI_STORE, lm, st));
  }
  return SPEC_OK;
}

int need_ctx(spec_ctx* c) { return c ? SPEC_OK : SPEC_E_INVAL; }

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
  if (c->len_hi + need > c->cap) return fail(c, SPEC_E_RANGE, "context would overflow the cache");
  return SPEC_OK;
}


// The kernels of one draft_step: k forwards of the draft model at one row (two rows for
// the first: the tokens at L-1 and L), each followed by truncation and a sampled draft.
int enqueue_draft(spec_ctx* c, int batch, int k, int32_t* draft_tok, const spec_probs& q) {
  Model& m = c->draft;
  const spec_sampler& s = c->cfg.sampler;
  const int V = m.d.vocab;
  const int P = 16 * m.mi;
  for (int j = 1; j <= k; ++j) {
    int rc;
    if (j == 1) {
      rc = forward(c, m, batch, 2, c->prev_tok, 1, c->last_tok, 1, -1, m.logits);
      if (rc) return rc;
      LAUNCH(c, P + PROF_TRUNC, launch_truncate(m.logits + V, SPEC_DTYPE_F32, batch, V, 2 * (int64_t)V, s, q, k,
                                                nullptr, c->trunc, c->stream));
    } else {
      rc = forward(c, m, batch, 1, draft_tok + (j - 2), k, nullptr, 0, j - 1, m.logits);
      if (rc) return rc;
      LAUNCH(c, P + PROF_TRUNC, launch_truncate(m.logits, SPEC_DTYPE_F32, batch, V, V, s, offset_rows(q, j - 1), k,
                                                nullptr, c->trunc, c->stream));
    }
    LAUNCH(c, P + PROF_SAMPLE, launch_sample(offset_rows(q, j - 1), k, batch, 1, j, c->cfg.seed, c->round_dev,
                                             0u, STREAM_DRAFT, draft_tok + (j - 1), k, nullptr, c->stream));
  }
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
  LAUNCH(c, PROF_TRUNC, launch_truncate(lg, SPEC_DTYPE_F32, batch * (k + 1), V, V, c->cfg.sampler, p, 1, nullptr,
                                        c->trunc, c->stream));
  return SPEC_OK;
}

// Runs `enqueue` directly, or through a captured graph: the first call with a given
// (kind, batch, k, buffer addresses) captures the launches on the context stream, later
// calls replay them.  Every kernel reads lengths and the round from device memory, so a
// replay computes exactly what a direct enqueue would.
template <typename F>
int run_graphed(spec_ctx* c, int kind, int batch, int k, const void* const key[8], F enqueue) {
  if (c->prof || !c->graphs || c->stream == nullptr) return enqueue();
  for (auto& g : c->gcache) {
    if (g.kind == kind && g.batch == batch && g.k == k && !memcmp(g.ptrs, key, sizeof g.ptrs)) {
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
  g.kind = kind;
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
  if (rc) {
    delete c;
    return rc;
  }
  c->target.layers.assign(cfg->target.layers, cfg->target.layers + cfg->target.n_layers);
  c->target.d.layers = nullptr;
  if (c->draft.present) {
    c->draft.layers.assign(cfg->draft.layers, cfg->draft.layers + cfg->draft.n_layers);
    c->draft.d.layers = nullptr;
  }
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
  if (e != hipSuccess) {
    delete c;
    return fail(nullptr, SPEC_E_HIP, "init kernels: %s", hipGetErrorString(e));
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
  Model* m = which == 0 ? &c->target : (which == 1 && c->draft.present ? &c->draft : nullptr);
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

int spec_set_last(spec_ctx* c, const int32_t* last_tok, const int32_t* prev_tok, const float* hidden,
                  int32_t batch) {
  (void)hidden;
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (!last_tok) return fail(c, SPEC_E_INVAL, "null last_tok");
  if (batch < 1 || batch > c->cfg.max_batch) return fail(c, SPEC_E_RANGE, "batch %d", batch);
  if (c->draft.present && !prev_tok) return fail(c, SPEC_E_INVAL, "a draft model needs prev_tok");
  if (c->phase != IDLE && c->phase != READY) return fail(c, SPEC_E_STATE, "set_last inside a cycle");
  if (!c->started) return fail(c, SPEC_E_STATE, "set_last needs a loaded cache prefix");
  HIPCHK(c, launch_copy_rows(last_tok, 1, c->last_tok, batch, c->stream));
  if (prev_tok) HIPCHK(c, launch_copy_rows(prev_tok, 1, c->prev_tok, batch, c->stream));
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
  int done = 0;
  while (done < P - 1) {
    const int chunk = std::min(std::min(c->target.mseq_max, P - 1 - done),
                               c->draft.present ? c->draft.mseq_max : 1 << 30);
    int rc = forward(c, c->target, batch, chunk, tokens + done, P, tokens + done + 1, P, 0, nullptr);
    if (rc) return rc;
    if (c->draft.present) {
      rc = forward(c, c->draft, batch, chunk, tokens + done, P, tokens + done + 1, P, 0, nullptr);
      if (rc) return rc;
    }
    HIPCHK(c, launch_add_len(c->len, batch, chunk, c->stream));
    done += chunk;
  }
  HIPCHK(c, launch_copy_rows(tokens + (P - 1), P, c->last_tok, batch, c->stream));
  if (P >= 2) HIPCHK(c, launch_copy_rows(tokens + (P - 2), P, c->prev_tok, batch, c->stream));
  c->len_lo = c->len_hi = L0 + P - 1;
  c->started = true;
  c->phase = READY;
  return SPEC_OK;
}

int draft_step(spec_ctx* c, int32_t batch, int32_t k, uint64_t round, int32_t* draft_tok, spec_probs* q,
               int32_t* n_drafted) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (c->cfg.draft_kind != SPEC_DRAFT_MODEL) return fail(c, SPEC_E_UNSUPPORTED, "no draft model configured");
  if (batch < 1 || batch > c->cfg.max_batch) return fail(c, SPEC_E_RANGE, "batch %d", batch);
  if (k < 1 || k > c->cfg.max_k) return fail(c, SPEC_E_RANGE, "k %d not in 1..max_k", k);
  if (!draft_tok) return fail(c, SPEC_E_INVAL, "null draft_tok");
  int rc = check_probs(c, q, "q", list_cap(c->cfg.sampler));
  if (rc) return rc;
  if (c->phase != READY) return fail(c, SPEC_E_STATE, "draft_step needs a start (prefill / set_last) or a trimmed cycle");
  if (c->len_lo < 1) return fail(c, SPEC_E_STATE, "draft model needs a token before the last one");
  rc = ensure_room(c, batch, k + 1);
  if (rc) return rc;
  HIPCHK(c, launch_set_u32(c->round_dev, (uint32_t)round, c->stream));
  const spec_probs qq = *q;
  const void* key[8] = {draft_tok, qq.ids, qq.probs, qq.count, (const void*)(intptr_t)qq.cap,
                        nullptr, nullptr, nullptr};
  rc = run_graphed(c, 1, batch, k, key, [&]() { return enqueue_draft(c, batch, k, draft_tok, qq); });
  if (rc) return rc;
  if (n_drafted) *n_drafted = k;
  c->phase = DRAFTED;
  c->phase_k = k;
  c->phase_batch = batch;
  return SPEC_OK;
}

int verify_step(spec_ctx* c, const int32_t* draft_tok, int32_t batch, int32_t k, float* logits_out,
                spec_probs* p) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (batch < 1 || batch > c->cfg.max_batch) return fail(c, SPEC_E_RANGE, "batch %d", batch);
  if (k < 0 || k > c->cfg.max_k) return fail(c, SPEC_E_RANGE, "k %d not in 0..max_k", k);
  if (k > 0 && !draft_tok) return fail(c, SPEC_E_INVAL, "null draft_tok");
  int rc = check_probs(c, p, "p", list_cap(c->cfg.sampler));
  if (rc) return rc;
  if (c->phase != READY && c->phase != DRAFTED)
    return fail(c, SPEC_E_STATE, "verify_step needs a start (prefill / set_last) or a trimmed cycle");
  rc = ensure_room(c, batch, k + 1);
  if (rc) return rc;
  const spec_probs pp = *p;
  const void* key[8] = {draft_tok, logits_out, pp.ids, pp.probs, pp.count, (const void*)(intptr_t)pp.cap,
                        nullptr, nullptr};
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
  LAUNCH(c, PROF_ACCEPT, launch_accept(a, c->stream));
  c->phase = ACCEPTED;
  return SPEC_OK;
}

int kv_trim(spec_ctx* c, const int32_t* n_acc, int32_t batch) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  if (c->phase != ACCEPTED) return fail(c, SPEC_E_STATE, "kv_trim must follow accept");
  if (batch != c->phase_batch) return fail(c, SPEC_E_STATE, "batch differs from the cycle");
  if (!n_acc) return fail(c, SPEC_E_INVAL, "null n_acc");
  LAUNCH(c, PROF_TRIM, launch_trim(c->len, n_acc, batch, c->stream));
  c->len_lo += 1;
  c->len_hi += 1 + c->phase_k;
  c->phase = READY;
  return SPEC_OK;
}

int spec_profile(spec_ctx* c, int32_t enable) {
  if (need_ctx(c)) return SPEC_E_INVAL;
  c->prof = enable != 0;
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
    launches[r.slot] += 1;
    c->ev_free.push_back(r.a);
    c->ev_free.push_back(r.b);
  }
  c->recs.clear();
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
  return SPEC_OK;
}

int spec_get_lengths(spec_ctx* c, int32_t* lengths, int32_t batch) {
  if (need_ctx(c) || !lengths) return SPEC_E_INVAL;
  if (batch < 1 || batch > c->cfg.max_batch) return fail(c, SPEC_E_RANGE, "batch %d", batch);
  HIPCHK(c, hipMemcpyAsync(lengths, c->len, sizeof(int32_t) * batch, hipMemcpyDeviceToHost, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
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

int spec_philox_uniforms(uint64_t seed, const uint32_t* ctr, int32_t n, float* out, void* stream) {
  if (!ctr || !out || n < 0) return SPEC_E_INVAL;
  return launch_philox(seed, ctr, n, out, (hipStream_t)stream) == hipSuccess ? SPEC_OK : SPEC_E_HIP;
}

int spec_ngram_match(const int32_t* ctx, const int32_t* lengths, int32_t batch, int32_t ld, int32_t k,
                     int32_t n_min, int32_t max_match, int32_t* drafts, int32_t* n_found, int32_t* match,
                     void* stream) {
  if (!ctx || !lengths || !drafts || !n_found || !match) return SPEC_E_INVAL;
  if (batch < 0 || ld < 1 || k < 1 || n_min < 1 || max_match < n_min) return SPEC_E_INVAL;
  NgramArgs a{ctx, lengths, batch, ld, k, n_min, max_match, drafts, n_found, match};
  return launch_ngram(a, (hipStream_t)stream) == hipSuccess ? SPEC_OK : SPEC_E_HIP;
}

}  // extern "C"
