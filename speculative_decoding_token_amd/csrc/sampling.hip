// Truncation, sampling, accept and n-gram kernels.
//
// Truncation ("Qwen3.5 and Qwen3.6 MTP head reaches 1.4x on Apple Silicon after three
// fixes", section "Truncation has to match on both sides": the same top_k / top_p on the
// draft and the verify side) runs in two launches:
//   1. topk_segment: a workgroup per (row, segment of <= 16384 logits) finds the segment's
//      exact top-k by the order (larger value, then lower id) from values held in
//      registers: the k-th largest per-thread maximum bounds the answer from below, the
//      elements at or above it are gathered into LDS and bitonic-sorted (a 64-step binary
//      search on the key replaces the gather when more than 1024 elements qualify, e.g.
//      on long runs of equal logits);
//   2. truncate_finish: a wavefront per row merges the segment lists, then one lane does
//      the float32 softmax, the top_p walk and the renormalization in the stated
//      sequential order, and the lanes write the kept pairs in ascending id order.
// Accept ("... after three fixes", section "The verify was wrong under sampling") keeps a
// draft with probability min(1, p/q) and replaces the first rejected one by a draw from
// max(0, p - q) renormalized; at temperature 0 it compares with the target's argmax
// ("What is Speculative Decoding and How Does a Draft Model Work?", section "#3").
// Every running sum here is a plain sequential float32 sum; no contraction into FMA.
#pragma clang fp contract(off)

#include "kernels.h"

namespace spec {

constexpr int TK_THREADS = 256;
constexpr int TK_EPT = 32;                      // logits held per thread
constexpr int TK_SEG = TK_THREADS * TK_EPT;     // longest segment
constexpr int TK_CAND = 1024;                   // LDS candidate slots
constexpr int FIN_THREADS = 256;
constexpr int FIN_SLOTS = 2048;                 // nseg * ksel must fit

// ---------------------------------------------------------------- block helpers
template <int N>
SPEC_DEVINL void bitonic_desc(uint64_t* s, int n_pow2) {
  for (int k = 2; k <= n_pow2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n_pow2; i += N) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t a = s[i], b = s[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (a < b) : (a > b)) {
            s[i] = b;
            s[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

SPEC_DEVINL int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

SPEC_DEVINL uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64), hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}
SPEC_DEVINL uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = __shfl((uint32_t)v, src, 64), hi = __shfl((uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Sorts one key per lane of a wavefront, descending: afterwards lane j holds the j-th largest.
SPEC_DEVINL uint64_t wave_sort_desc(uint64_t v, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t o = shfl_xor_u64(v, j);
      const bool up = (lane & j) == 0;          // lower partner of the pair
      const bool desc = (lane & k) == 0;        // this run sorts descending
      const bool keep_max = (up == desc);
      v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
    }
  }
  return v;
}

// ---------------------------------------------------------------- 1. segment top-k
// Output: the segment's ksel largest keys, descending, zero-padded.
template <int DT, bool VEC>
__global__ __launch_bounds__(TK_THREADS) void topk_segment_kernel(TruncArgs a) {
  constexpr int VW = (DT == SPEC_DTYPE_BF16) ? 8 : 4;  // elements per 16-byte load
  constexpr int NV = TK_EPT / VW;
  __shared__ uint64_t sk[TK_CAND];
  __shared__ uint64_t s_wt[TK_THREADS / 64];
  __shared__ int s_wcnt[TK_THREADS / 64];
  __shared__ int s_bad, s_total;
  __shared__ unsigned long long s_count;

  const int row = blockIdx.y, seg = blockIdx.x, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int s0 = seg * a.seg_len;
  const int s1 = min(s0 + a.seg_len, a.vocab);
  const float T = a.temperature;
  const bool scale = T > 0.0f;
  if (t == 0) s_bad = 0;

  // all loads first, addresses clamped into the row
  const char* base = (const char*)a.logits;
  const int64_t rowoff = (int64_t)row * a.stride;
  float x[TK_EPT];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int i0 = s0 + (v * TK_THREADS + t) * VW;
    if (VEC) {
      const int ic = min(i0, a.vocab - VW);
      if (DT == SPEC_DTYPE_BF16) {
        const uint4 w = *(const uint4*)(base + (rowoff + ic) * 2);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[v * VW + 2 * e] = __uint_as_float(ww[e] << 16);
          x[v * VW + 2 * e + 1] = __uint_as_float(ww[e] & 0xFFFF0000u);
        }
      } else {
        const float4 w = *(const float4*)(base + (rowoff + ic) * 4);
        x[v * VW + 0] = w.x; x[v * VW + 1] = w.y; x[v * VW + 2] = w.z; x[v * VW + 3] = w.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        const int ic = min(i0 + e, a.vocab - 1);
        x[v * VW + e] = (DT == SPEC_DTYPE_BF16) ? bf16_to_f32(((const bf16_t*)base)[rowoff + ic])
                                                : ((const float*)base)[rowoff + ic];
      }
    }
  }
  bool bad = false;
  uint64_t tmax = 0;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < VW; ++e) {
      const int i = s0 + (v * TK_THREADS + t) * VW + e;
      float z = x[v * VW + e];
      if (i < s1) {
        if (__builtin_isnan(z) || z == __builtin_inff()) bad = true;
        if (scale) z = z / T;
      } else {
        z = __builtin_nanf("");  // outside the segment: never a candidate
      }
      x[v * VW + e] = z;
      if (!__builtin_isnan(z)) {
        const uint64_t k = order_key(z, (uint32_t)i);
        tmax = k > tmax ? k : tmax;
      }
    }
  __syncthreads();
  if (bad) atomicOr(&s_bad, 1);

  // lower bound: each wave's ceil(ksel/4)-th largest thread maximum; the smallest of the
  // four leaves at least ksel elements at or above it
  const int kw = (a.ksel + 3) / 4;
  const uint64_t srt = wave_sort_desc(tmax, lane);
  const uint64_t wt = shfl_u64(srt, kw - 1);
  if (lane == 0) s_wt[wave] = wt;
  __syncthreads();
  uint64_t tau = s_wt[0];
#pragma unroll
  for (int w = 1; w < TK_THREADS / 64; ++w) tau = s_wt[w] < tau ? s_wt[w] : tau;

  int cnt = 0;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < VW; ++e) {
      const float z = x[v * VW + e];
      const int i = s0 + (v * TK_THREADS + t) * VW + e;
      if (!__builtin_isnan(z) && order_key(z, (uint32_t)i) >= tau) ++cnt;
    }
  // block exclusive scan of the counts: wave scan by shuffles, wave totals through LDS
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_wcnt[wave] = incl;
  __syncthreads();
  int woff = 0, total = 0;
#pragma unroll
  for (int w = 0; w < TK_THREADS / 64; ++w) {
    if (w < wave) woff += s_wcnt[w];
    total += s_wcnt[w];
  }
  uint64_t* out = a.part + ((int64_t)row * a.nseg + seg) * a.ksel;

  if (total <= TK_CAND) {
    int off = woff + incl - cnt;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        const float z = x[v * VW + e];
        const int i = s0 + (v * TK_THREADS + t) * VW + e;
        if (!__builtin_isnan(z)) {
          const uint64_t k = order_key(z, (uint32_t)i);
          if (k >= tau) sk[off++] = k;
        }
      }
    __syncthreads();
    if (total <= 256) {
      // rank selection: a candidate's rank is the number of larger candidates (keys are unique)
      for (int c = t; c < total; c += TK_THREADS) {
        const uint64_t k = sk[c];
        int rank = 0;
        for (int o = 0; o < total; ++o) rank += sk[o] > k;
        if (rank < a.ksel) out[rank] = k;
      }
    } else {
      const int p2 = next_pow2(total);
      for (int i = total + t; i < p2; i += TK_THREADS) sk[i] = 0;
      __syncthreads();
      bitonic_desc<TK_THREADS>(sk, p2);
      for (int i = t; i < a.ksel; i += TK_THREADS) out[i] = sk[i];
    }
    for (int i = total + t; i < a.ksel; i += TK_THREADS) out[i] = 0;
  } else {
    // exact ksel-th largest key by binary search over the 64-bit key space
    uint64_t lo = 0, hi = ~0ull;
    while (lo < hi) {
      const uint64_t mid = lo + (hi - lo) / 2 + 1;
      if (t == 0) s_count = 0;
      __syncthreads();
      int c = 0;
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < VW; ++e) {
          const float z = x[v * VW + e];
          const int i = s0 + (v * TK_THREADS + t) * VW + e;
          if (!__builtin_isnan(z) && order_key(z, (uint32_t)i) >= mid) ++c;
        }
      if (c) atomicAdd(&s_count, (unsigned long long)c);
      __syncthreads();
      const bool enough = s_count >= (unsigned long long)a.ksel;
      __syncthreads();
      if (enough) lo = mid; else hi = mid - 1;
    }
    if (t == 0) s_total = 0;
    for (int i = t; i < TK_CAND; i += TK_THREADS) sk[i] = 0;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        const float z = x[v * VW + e];
        const int i = s0 + (v * TK_THREADS + t) * VW + e;
        if (!__builtin_isnan(z)) {
          const uint64_t k = order_key(z, (uint32_t)i);
          if (k >= lo) {
            const int slot = atomicAdd(&s_total, 1);
            if (slot < TK_CAND) sk[slot] = k;
          }
        }
      }
    __syncthreads();
    const int p2 = next_pow2(max(a.ksel, 2));
    bitonic_desc<TK_THREADS>(sk, p2);
    for (int i = t; i < a.ksel; i += TK_THREADS) out[i] = sk[i];
  }
  if (t == 0) a.bad[(int64_t)row * a.nseg + seg] = (uint8_t)(s_bad ? 1 : 0);
}

// ---------------------------------------------------------------- 2. finish
// Merges the sorted segment lists by rank (a key's rank = its index in its own list plus
// the number of larger keys in every other list, found by binary search), then lane 0
// does the float32 softmax / top_p / renormalization in the stated sequential order.
__global__ __launch_bounds__(FIN_THREADS) void truncate_finish_kernel(TruncArgs a, spec_probs out,
                                                                      int out_rs, float top_p,
                                                                      uint8_t* flags) {
  __shared__ uint64_t sk[FIN_SLOTS];
  __shared__ uint64_t top[SPEC_TOPK_MAX];
  __shared__ float s_p[SPEC_TOPK_MAX];
  __shared__ int s_id[SPEC_TOPK_MAX];
  __shared__ int s_n, s_bad;
  const int row = blockIdx.x, t = threadIdx.x;
  const int K = a.ksel, nk = a.nseg * K;
  const uint64_t* src = a.part + (int64_t)row * nk;
  for (int i = t; i < nk; i += FIN_THREADS) sk[i] = src[i];
  for (int i = t; i < K; i += FIN_THREADS) top[i] = 0;
  if (t == 0) {
    int b = 0;
    for (int s = 0; s < a.nseg; ++s) b |= a.bad[(int64_t)row * a.nseg + s];
    s_bad = b;
  }
  __syncthreads();
  for (int c = t; c < nk; c += FIN_THREADS) {
    const uint64_t key = sk[c];
    if (key == 0) continue;
    const int own = c / K;
    int rank = c % K;
    for (int s = 0; s < a.nseg && rank < K; ++s) {
      if (s == own) continue;
      const uint64_t* l = sk + s * K;
      int lo = 0, hi = K;  // first index whose key is smaller (empty slots are 0)
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (l[mid] > key) lo = mid + 1; else hi = mid;
      }
      rank += lo;
    }
    if (rank < K) top[rank] = key;
  }
  __syncthreads();

  if (t == 0) {
    uint8_t fl = 0;
    int n = 0;
    if (!s_bad) {
      for (int i = 0; i < K; ++i) {
        const uint64_t key = top[i];
        if (key == 0) break;
        const float zi = key_value(key);
        if (zi == -__builtin_inff()) break;  // sorted: the rest is -inf or empty
        s_id[n] = (int)key_id(key);
        s_p[n] = zi;
        ++n;
      }
    }
    if (n == 0) {
      fl |= SPEC_FLAG_BAD_ROW;
    } else if (!(a.temperature > 0.0f)) {
      n = 1;
      s_p[0] = 1.0f;
    } else {
      const float m = s_p[0];
      float S = 0.0f;
      for (int i = 0; i < n; ++i) {
        s_p[i] = expf(s_p[i] - m);
        S = S + s_p[i];
      }
      for (int i = 0; i < n; ++i) s_p[i] = s_p[i] / S;
      int nkeep = n;
      if (top_p < 1.0f) {
        float excl = 0.0f, excl_last = 0.0f;
        nkeep = 0;
        for (int i = 0; i < n; ++i) {
          if (i > 0 && !(excl < top_p)) break;
          excl_last = excl;
          ++nkeep;
          excl = excl + s_p[i];
        }
        float margin = __builtin_inff();
        if (nkeep > 1) margin = fminf(margin, fabsf(excl_last - top_p));
        if (nkeep < n) margin = fminf(margin, fabsf(excl - top_p));
        if (margin < NEAR_TIE) fl |= SPEC_FLAG_TOPP_TIE;
      }
      float Z = 0.0f;
      for (int i = 0; i < nkeep; ++i) Z = Z + s_p[i];
      for (int i = 0; i < nkeep; ++i) s_p[i] = s_p[i] / Z;
      n = nkeep;
    }
    s_n = n;
    out.count[(int64_t)row * out_rs] = n;
    if (flags) flags[row] = fl;
  }
  __syncthreads();
  const int n = s_n;
  if (t < n) {
    const int my = s_id[t];
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += s_id[j] < my;
    const int64_t orow = (int64_t)row * out_rs;
    out.ids[orow * out.cap + rank] = my;
    out.probs[orow * out.cap + rank] = s_p[t];
  }
}

// ---------------------------------------------------------------- sampling from a list
// First id (ascending) whose running sum exceeds u * Z; else the last id with mass.
SPEC_DEVINL int sample_list(const int32_t* ids, const float* w, int n, float u, uint8_t* fl) {
  if (n <= 0) {
    *fl |= SPEC_FLAG_BAD_ROW;
    return -1;
  }
  float Z = 0.0f;
  for (int i = 0; i < n; ++i) Z = Z + w[i];
  const float thr = u * Z;
  float c = 0.0f, cprev = 0.0f;
  int pick = -1;
  for (int i = 0; i < n; ++i) {
    cprev = c;
    c = c + w[i];
    if (c > thr) {
      pick = i;
      break;
    }
  }
  if (pick < 0) {
    for (int i = n - 1; i >= 0; --i)
      if (w[i] > 0.0f) {
        pick = i;
        break;
      }
    if (pick < 0) pick = n - 1;
    // recompute the running sums at the chosen step
    c = 0.0f;
    cprev = 0.0f;
    for (int i = 0; i <= pick; ++i) {
      cprev = c;
      c = c + w[i];
    }
  }
  float margin = fabsf(c - thr);
  if (pick > 0) margin = fminf(margin, fabsf(cprev - thr));
  if (margin < NEAR_TIE) *fl |= SPEC_FLAG_SAMPLE_TIE;
  return ids[pick];
}

__global__ void sample_kernel(spec_probs lists, int list_rs, int rows, int per_seq, int slot_base,
                              uint64_t seed, const uint32_t* rnd_ptr, uint32_t rnd_val,
                              uint32_t stream_id, int32_t* tokens, int tok_ld, uint8_t* flags) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const int64_t lr = (int64_t)r * list_rs;
  const int n = min(lists.count[lr], lists.cap);
  const int seq = r / per_seq, jj = r % per_seq;
  uint8_t fl = 0;
  int tok = -1;
  if (n <= 0) {
    fl |= SPEC_FLAG_BAD_ROW;
  } else {
    const uint32_t rnd = rnd_ptr ? *rnd_ptr : rnd_val;
    const float u = philox_uniform(seed, (uint32_t)(slot_base + jj), rnd, (uint32_t)seq, stream_id);
    tok = sample_list(lists.ids + lr * lists.cap, lists.probs + lr * lists.cap, n, u, &fl);
  }
  tokens[(int64_t)seq * tok_ld + jj] = tok;
  if (flags) flags[r] = fl;
}

// ---------------------------------------------------------------- accept
SPEC_DEVINL float list_prob(const int32_t* ids, const float* p, int n, int tok) {
  for (int i = 0; i < n; ++i)
    if (ids[i] == tok) return p[i];
  return 0.0f;
}
// count of a list row, clamped to what the row can hold
SPEC_DEVINL int list_len(const spec_probs& l, int64_t row) {
  const int n = l.count[row];
  return n < 0 ? 0 : (n > l.cap ? l.cap : (n > SPEC_TOPK_MAX ? SPEC_TOPK_MAX : n));
}
SPEC_DEVINL int list_argmax(const int32_t* ids, const float* p, int n) {
  int best = 0;
  for (int i = 1; i < n; ++i)
    if (p[i] > p[best]) best = i;  // ids ascending: the first maximum has the lowest id
  return ids[best];
}

__global__ void accept_kernel(AcceptArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.batch) return;
  const int k = a.k;
  // drafts actually proposed for this sequence (an n-gram lookup may find fewer than k);
  // the rows past them are not tested and the bonus comes from row kb
  const int kb = a.kcap ? min(max(a.kcap[b], 0), k) : k;
  const int32_t* d = a.drafts + (int64_t)b * k;
  int32_t* out = a.out_tok + (int64_t)b * (k + 1);
  uint8_t fl = 0;
  int n = kb;
  int emitted = -1;
  bool stopped = false;  // a draft was rejected, or its target row was empty
  for (int j = 0; j < kb; ++j) {
    const int64_t pr = (int64_t)b * (k + 1) + j, qr = (int64_t)b * k + j;
    const int32_t* pid = a.p.ids + pr * a.p.cap;
    const float* pp = a.p.probs + pr * a.p.cap;
    const int pn = list_len(a.p, pr);
    if (pn <= 0) {
      // no distribution to test draft j against (its logits held no finite value): nothing
      // from j on is kept and no token is emitted (-1 signals the bad row)
      fl |= SPEC_FLAG_BAD_ROW;
      n = j;
      stopped = true;
      break;
    }
    if (a.greedy) {
      const int am = list_argmax(pid, pp, pn);
      if (d[j] == am) {
        out[j] = d[j];
        continue;
      }
      n = j;
      emitted = am;
      stopped = true;
      break;
    }
    const int32_t* qid = a.q.ids + qr * a.q.cap;
    const float* qp = a.q.probs + qr * a.q.cap;
    const int qn = list_len(a.q, qr);
    const float pj = list_prob(pid, pp, pn, d[j]);
    const float qj = list_prob(qid, qp, qn, d[j]);
    const float ratio = pj / qj;
    const float u = philox_uniform(a.seed, (uint32_t)(j + 1), a.round, (uint32_t)b, STREAM_ACCEPT);
    if (__builtin_isfinite(ratio) && fabsf(u - ratio) < NEAR_TIE) fl |= SPEC_FLAG_ACCEPT_TIE;
    if (u < ratio) {
      out[j] = d[j];
      continue;
    }
    // residual max(0, p - q) over p's support, ascending ids (both lists are ascending)
    float r[SPEC_TOPK_MAX];
    float Z = 0.0f;
    int qi = 0;
    for (int i = 0; i < pn; ++i) {
      while (qi < qn && qid[qi] < pid[i]) ++qi;
      const float qv = (qi < qn && qid[qi] == pid[i]) ? qp[qi] : 0.0f;
      const float diff = pp[i] - qv;
      r[i] = diff > 0.0f ? diff : 0.0f;
      Z = Z + r[i];
    }
    const float ur = philox_uniform(a.seed, 0u, a.round, (uint32_t)b, STREAM_RESIDUAL);
    emitted = (Z > 0.0f) ? sample_list(pid, r, pn, ur, &fl) : sample_list(pid, pp, pn, ur, &fl);
    n = j;
    stopped = true;
    break;
  }
  if (!stopped) {
    // every draft kept: bonus token from the target row after the last draft
    const int64_t pr = (int64_t)b * (k + 1) + kb;
    const int32_t* pid = a.p.ids + pr * a.p.cap;
    const float* pp = a.p.probs + pr * a.p.cap;
    const int pn = list_len(a.p, pr);
    if (pn <= 0) {
      fl |= SPEC_FLAG_BAD_ROW;
      emitted = -1;
    } else if (a.greedy) {
      emitted = list_argmax(pid, pp, pn);
    } else {
      const float ur = philox_uniform(a.seed, 0u, a.round, (uint32_t)b, STREAM_RESIDUAL);
      emitted = sample_list(pid, pp, pn, ur, &fl);
    }
    n = kb;
  }
  out[n] = emitted;
  a.n_acc[b] = n;
  if (a.near_tie) a.near_tie[b] = fl;
  // a bad last row leaves -1 in out_tok as the signal; the context state keeps token 0
  const int32_t kept = emitted < 0 ? 0 : emitted;
  if (a.last_tok) {
    // the token now at position L+n becomes the previous token, the emitted one the last
    a.prev_tok[b] = (n == 0) ? a.last_tok[b] : d[n - 1];
    a.last_tok[b] = kept;
  }
  if (a.hist) {
    int32_t* h = a.hist + (int64_t)b * a.hist_ld + a.len[b] + 1;
    for (int i = 0; i < n; ++i) h[i] = d[i];
    h[n] = kept;
  }
  if (a.stats) {
    if (b == 0) atomicAdd((unsigned long long*)&a.stats[0], 1ull);
    atomicAdd((unsigned long long*)&a.stats[1], (unsigned long long)kb);
    atomicAdd((unsigned long long*)&a.stats[2], (unsigned long long)n);
    atomicAdd((unsigned long long*)&a.stats[3], (unsigned long long)(n + 1));
  }
}

// ---------------------------------------------------------------- kv trim
// n_acc[b] is clamped to [0, k]: the host's bound on the lengths assumes at most k drafts kept.
__global__ void trim_kernel(int32_t* len, const int32_t* n_acc, int batch, int k, int32_t* mlen) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  // the MTP layer keeps its entries up to the old last position: later ones were built from
  // its own hidden states rather than the target's
  if (mlen) mlen[b] = min(mlen[b], len[b] + 1);
  len[b] += 1 + min(max(n_acc[b], 0), k);
}

// ---------------------------------------------------------------- token history
__global__ void onehot_kernel(const int32_t* drafts, int rows, spec_probs q) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  q.ids[(int64_t)r * q.cap] = drafts[r];
  q.probs[(int64_t)r * q.cap] = 1.0f;
  q.count[r] = 1;
}

__global__ void hist_write_kernel(int32_t* hist, int ld, const int32_t* src, int src_ld, int batch, int n,
                                  int pos0) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= (int64_t)batch * n) return;
  const int b = (int)(i / n), j = (int)(i % n);
  hist[(int64_t)b * ld + pos0 + j] = src[(int64_t)b * src_ld + j];
}

__global__ void hist_set_last_kernel(int32_t* hist, int ld, const int32_t* len, const int32_t* last,
                                     const int32_t* prev, int batch) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int L = len[b];
  hist[(int64_t)b * ld + L] = last[b];
  if (prev && L >= 1) hist[(int64_t)b * ld + L - 1] = prev[b];
}

__global__ void set_u32_kernel(uint32_t* p, uint32_t v) { *p = v; }

hipError_t launch_set_u32(uint32_t* p, uint32_t v, hipStream_t st) {
  hipLaunchKernelGGL(set_u32_kernel, dim3(1), dim3(1), 0, st, p, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------- Philox uniforms
__global__ void philox_kernel(uint64_t seed, const uint32_t* ctr, int n, float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint4 c = make_uint4(ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]);
  const uint4 o = philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  out[i] = (float)(o.x >> 8) * (1.0f / 16777216.0f);
}

// ---------------------------------------------------------------- n-gram lookup
// "Speculative decoding on Apple Silicon" (OptiQ docs), section "N-gram lookup: any
// model": when the last tokens match an earlier stretch of the context, the tokens that
// followed it are drafted.  One workgroup per sequence; a thread per earlier end position.
__global__ __launch_bounds__(256) void ngram_kernel(NgramArgs a) {
  __shared__ unsigned long long s_best;
  const int b = blockIdx.x, t = threadIdx.x;
  const int32_t* c = a.ctx + (int64_t)b * a.ld;
  const int n = min(max(a.lengths[b] + a.len_add, 0), a.ld);
  if (t == 0) s_best = 0;
  __syncthreads();
  unsigned long long best = 0;
  for (int e = t; e < n - 1; e += blockDim.x) {
    int ell = 0;
    while (ell < a.max_match && e - ell >= 0 && c[e - ell] == c[n - 1 - ell]) ++ell;
    if (ell >= a.n_min) {
      const unsigned long long key = ((unsigned long long)ell << 32) | (unsigned)e;
      best = key > best ? key : best;
    }
  }
  if (best) atomicMax(&s_best, best);
  __syncthreads();
  if (t == 0) {
    const unsigned long long bk = s_best;
    int32_t* d = a.drafts + (int64_t)b * a.k;
    int found = 0;
    int last = n > 0 ? c[n - 1] : 0;
    if (bk) {
      const int e = (int)(bk & 0xFFFFFFFFu);
      const int ell = (int)(bk >> 32);
      for (int i = 0; i < a.k && e + 1 + i <= n - 1; ++i) {
        last = c[e + 1 + i];
        d[i] = last;
        ++found;
      }
      a.match[2 * b] = ell;
      a.match[2 * b + 1] = e;
    } else {
      a.match[2 * b] = 0;
      a.match[2 * b + 1] = -1;
    }
    for (int i = found; i < a.k; ++i) d[i] = last;
    a.n_found[b] = found;
  }
}

// ---------------------------------------------------------------- launchers
int truncate_scratch_bytes(int rows, int vocab, size_t* bytes) {
  const int nseg = (vocab + TK_SEG - 1) / TK_SEG;
  if (nseg * SPEC_TOPK_MAX > FIN_SLOTS) return SPEC_E_UNSUPPORTED;
  *bytes = (size_t)rows * nseg * SPEC_TOPK_MAX * sizeof(uint64_t) + (size_t)rows * nseg + 256;
  return SPEC_OK;
}

hipError_t launch_truncate(const void* logits, int dtype, int rows, int vocab, int64_t stride,
                           const spec_sampler& s, const spec_probs& out, int out_rs, uint8_t* flags,
                           void* scratch, hipStream_t st) {
  TruncArgs a;
  a.logits = logits;
  a.stride = stride;
  a.vocab = vocab;
  a.rows = rows;
  a.temperature = s.temperature;
  a.ksel = s.temperature > 0.0f ? s.top_k : 1;
  a.nseg = (vocab + TK_SEG - 1) / TK_SEG;
  int seg = (vocab + a.nseg - 1) / a.nseg;
  a.seg_len = (seg + 7) / 8 * 8;
  a.part = (uint64_t*)scratch;
  a.bad = (uint8_t*)scratch + (size_t)rows * a.nseg * SPEC_TOPK_MAX * sizeof(uint64_t);
  if (rows == 0) return hipSuccess;
  const size_t esz = dtype == SPEC_DTYPE_BF16 ? 2 : 4;
  // 16-byte loads need aligned rows and a vocabulary that is a whole number of vectors
  const bool vec = ((uintptr_t)logits % 16 == 0) && ((stride * esz) % 16 == 0) && (vocab % (int)(16 / esz) == 0);
  dim3 g1(a.nseg, rows);
  if (dtype == SPEC_DTYPE_BF16) {
    if (vec) hipLaunchKernelGGL((topk_segment_kernel<SPEC_DTYPE_BF16, true>), g1, dim3(TK_THREADS), 0, st, a);
    else hipLaunchKernelGGL((topk_segment_kernel<SPEC_DTYPE_BF16, false>), g1, dim3(TK_THREADS), 0, st, a);
  } else {
    if (vec) hipLaunchKernelGGL((topk_segment_kernel<SPEC_DTYPE_F32, true>), g1, dim3(TK_THREADS), 0, st, a);
    else hipLaunchKernelGGL((topk_segment_kernel<SPEC_DTYPE_F32, false>), g1, dim3(TK_THREADS), 0, st, a);
  }
  hipLaunchKernelGGL(truncate_finish_kernel, dim3(rows), dim3(FIN_THREADS), 0, st, a, out, out_rs,
                     s.top_p, flags);
  return hipGetLastError();
}

hipError_t launch_sample(const spec_probs& lists, int list_rs, int rows, int per_seq, int slot_base,
                         uint64_t seed, const uint32_t* rnd_ptr, uint32_t rnd, uint32_t stream_id,
                         int32_t* tokens, int tok_ld, uint8_t* flags, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(sample_kernel, dim3((rows + 63) / 64), dim3(64), 0, st, lists, list_rs, rows,
                     per_seq, slot_base, seed, rnd_ptr, rnd, stream_id, tokens, tok_ld, flags);
  return hipGetLastError();
}

hipError_t launch_accept(const AcceptArgs& a, hipStream_t st) {
  if (a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(accept_kernel, dim3((a.batch + 63) / 64), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_trim(int32_t* len, const int32_t* n_acc, int batch, int k, int32_t* mlen, hipStream_t st) {
  hipLaunchKernelGGL(trim_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, len, n_acc, batch, k, mlen);
  return hipGetLastError();
}

hipError_t launch_onehot(const int32_t* drafts, int rows, const spec_probs& q, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(onehot_kernel, dim3((rows + 63) / 64), dim3(64), 0, st, drafts, rows, q);
  return hipGetLastError();
}

hipError_t launch_hist_write(int32_t* hist, int ld, const int32_t* src, int src_ld, int batch, int n, int pos0,
                             hipStream_t st) {
  const int64_t tot = (int64_t)batch * n;
  if (tot == 0) return hipSuccess;
  hipLaunchKernelGGL(hist_write_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, hist, ld, src,
                     src_ld, batch, n, pos0);
  return hipGetLastError();
}

hipError_t launch_hist_set_last(int32_t* hist, int ld, const int32_t* len, const int32_t* last,
                                const int32_t* prev, int batch, hipStream_t st) {
  hipLaunchKernelGGL(hist_set_last_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, hist, ld, len, last, prev,
                     batch);
  return hipGetLastError();
}

hipError_t launch_philox(uint64_t seed, const uint32_t* ctr, int n, float* out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(philox_kernel, dim3((n + 255) / 256), dim3(256), 0, st, seed, ctr, n, out);
  return hipGetLastError();
}

hipError_t launch_ngram(const NgramArgs& a, hipStream_t st) {
  if (a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(ngram_kernel, dim3(a.batch), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace spec
