// Truncation, sampling, accept and n-gram kernels.
//
// Truncation ("Qwen3.5 and Qwen3.6 MTP head reaches 1.4x on Apple Silicon after three
// fixes", section "Truncation has to match on both sides": the same top_k / top_p on the
// draft and the verify side) runs in two launches:
//   1. topk_segment: a workgroup per (row, segment of <= 16384 logits) finds the segment's
//      exact top-k by the order (larger value, then lower id) from values held in
//      registers: the k-th largest per-thread maximum of the raw values bounds the answer
//      from below, the few elements at or above it are gathered into LDS and ranked exactly
//      (a 64-step binary search on the key replaces the gather when more than 1024 elements
//      qualify, e.g. on long runs of equal logits, or when the division by the temperature
//      could tie the bound with the answer);
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
constexpr int TK_EPT = 64;                      // logits held per thread
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

// The largest 64-bit key of the wavefront in every lane: the moves of wave_max (common.h) applied
// to both halves of the key.
template <int CTRL>
SPEC_DEVINL uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
SPEC_DEVINL uint64_t wave_max_u64(uint64_t v) {
  auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  v = mx(v, dpp_u64<0xB1>(v));
  v = mx(v, dpp_u64<0x4E>(v));
  v = mx(v, dpp_u64<0x141>(v));
  v = mx(v, dpp_u64<0x140>(v));
  const auto l16 = __builtin_amdgcn_permlane16_swap((int)(uint32_t)v, (int)(uint32_t)v, false, false);
  const auto h16 = __builtin_amdgcn_permlane16_swap((int)(uint32_t)(v >> 32), (int)(uint32_t)(v >> 32), false, false);
  v = mx(((uint64_t)(uint32_t)h16[0] << 32) | (uint32_t)l16[0], ((uint64_t)(uint32_t)h16[1] << 32) | (uint32_t)l16[1]);
  const auto l32 = __builtin_amdgcn_permlane32_swap((int)(uint32_t)v, (int)(uint32_t)v, false, false);
  const auto h32 = __builtin_amdgcn_permlane32_swap((int)(uint32_t)(v >> 32), (int)(uint32_t)(v >> 32), false, false);
  return mx(((uint64_t)(uint32_t)h32[0] << 32) | (uint32_t)l32[0], ((uint64_t)(uint32_t)h32[1] << 32) | (uint32_t)l32[1]);
}

// ---------------------------------------------------------------- 1. segment top-k
// Raw keys: an integer order of the stored bits (larger value, larger key; -0 just below +0;
// NaN above +inf or below -inf by its sign), 16 bits for a bf16 value and 32 for a float32
// one.  They bound the candidates only; the exact order is order_key's.
constexpr uint32_t KEY16_NINF = 0x007Fu, KEY16_PINF = 0xFF80u;
constexpr uint32_t KEY32_NINF = 0x007FFFFFu, KEY32_PINF = 0xFF800000u;
typedef short i16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// Two bf16 values packed in a word -> their two 16-bit keys, packed the same way.
SPEC_DEVINL uint32_t raw_keys16x2(uint32_t w) {
  const i16x2_t sgn = __builtin_bit_cast(i16x2_t, w) >> (i16x2_t){15, 15};
  return w ^ (__builtin_bit_cast(uint32_t, sgn) | 0x80008000u);
}
SPEC_DEVINL uint32_t raw_key32(uint32_t u) {
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
// Inverse of the raw keys: the value as a float.
SPEC_DEVINL float key16_value(uint32_t k) {
  const uint32_t b = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
  return __uint_as_float(b << 16);
}
SPEC_DEVINL float key32_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Output: the segment's ksel largest keys (order of value / T, then lower id), descending,
// zero-padded.  Every thread holds TK_EPT logits and turns them into raw keys in place (bf16:
// two per word, with packed 16-bit arithmetic), keeping its largest and smallest key.  In each
// wavefront, a 16- or 32-step bitwise search over ballots finds the ceil(ksel / 4)-th largest
// thread maximum; the smallest of the four is a bound that at least ksel logits reach.  Only
// the logits reaching it go to LDS, with their ids, and are ordered exactly (value / T as an
// IEEE float32 division, then id).  Every logit below the bound is at most the value whose key
// precedes the bound's; after the division (which keeps the order of values but may make two
// equal) that value must stay below the ksel-th candidate, else, or with more than TK_CAND
// candidates, the segment is searched exhaustively.  NaN or +inf anywhere marks the row bad.
template <int DT, bool VEC>
__global__ __launch_bounds__(TK_THREADS) void topk_segment_kernel(TruncArgs a) {
  constexpr bool BF = DT == SPEC_DTYPE_BF16;
  constexpr int VW = BF ? 8 : 4;  // elements per 16-byte load
  constexpr int NV = TK_EPT / VW;
  constexpr int KB = BF ? 16 : 32;  // key bits
  __shared__ uint64_t sk[TK_CAND];
  __shared__ float s_cz[TK_CAND];
  __shared__ int s_ci[TK_CAND];
  __shared__ uint32_t s_wt[TK_THREADS / 64];
  __shared__ int s_bad, s_n, s_slow, s_total;
  __shared__ unsigned long long s_count;

  const int row = blockIdx.y, seg = blockIdx.x, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int s0 = seg * a.seg_len;
  const int s1 = min(s0 + a.seg_len, a.vocab);
  const float T = a.temperature;
  const bool scale = T > 0.0f;
  if (t == 0) {
    s_bad = 0;
    s_n = 0;
    s_slow = 0;
  }
  // all loads first; elements past the segment hold -inf (never bad, lowest order) and are
  // excluded by index wherever a candidate is taken
  const char* base = (const char*)a.logits;
  const int64_t rowoff = (int64_t)row * a.stride;
  uint32_t key[NV][4];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int i0 = s0 + (v * TK_THREADS + t) * VW;
    if (VEC) {
      const int ic = min(i0, a.vocab - VW);
      const uint4 r = *(const uint4*)(base + (rowoff + ic) * (BF ? 2 : 4));
      key[v][0] = r.x;
      key[v][1] = r.y;
      key[v][2] = r.z;
      key[v][3] = r.w;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (BF) {
          const int ia = min(i0 + 2 * q, a.vocab - 1), ib = min(i0 + 2 * q + 1, a.vocab - 1);
          const bf16_t* p = (const bf16_t*)base + rowoff;
          key[v][q] = (uint32_t)p[ia] | ((uint32_t)p[ib] << 16);
        } else {
          key[v][q] = __float_as_uint(((const float*)base)[rowoff + min(i0 + q, a.vocab - 1)]);
        }
      }
    }
  }
  if (a.skip && *a.skip) return;  // a skipped draft launch (argument fetched with the others)
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int i0 = s0 + (v * TK_THREADS + t) * VW;
    if (i0 + VW > s1) {
#pragma unroll
      for (int e = 0; e < VW; ++e)
        if (i0 + e >= s1) {
          if (BF) {
            uint32_t& w = key[v][e >> 1];
            w = (e & 1) ? ((w & 0xFFFFu) | 0xFF800000u) : ((w & 0xFFFF0000u) | 0xFF80u);
          } else {
            key[v][e] = 0xFF800000u;
          }
        }
    }
  }
  // pass 1: raw keys in place; the thread's largest and smallest
  uint32_t tmax, tmin;
  if (BF) {
    u16x2_t mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        key[v][q] = raw_keys16x2(key[v][q]);
        const u16x2_t kv = __builtin_bit_cast(u16x2_t, key[v][q]);
        mx = __builtin_elementwise_max(mx, kv);
        mn = __builtin_elementwise_min(mn, kv);
      }
    tmax = mx.x > mx.y ? mx.x : mx.y;
    tmin = mn.x < mn.y ? mn.x : mn.y;
    if (tmax >= KEY16_PINF || tmin < KEY16_NINF) atomicOr(&s_bad, 1);  // +inf or NaN
  } else {
    tmax = 0;
    tmin = 0xFFFFFFFFu;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        key[v][q] = raw_key32(key[v][q]);
        tmax = key[v][q] > tmax ? key[v][q] : tmax;
        tmin = key[v][q] < tmin ? key[v][q] : tmin;
      }
    if (tmax >= KEY32_PINF || tmin < KEY32_NINF) atomicOr(&s_bad, 1);
  }
  // the bound: per wavefront the largest x that at least ceil(ksel/4) thread maxima reach,
  // bit by bit from the top; the smallest over the four wavefronts
  const int kw = (a.ksel + 3) / 4;
  uint32_t wt = 0;
#pragma unroll
  for (int b = KB - 1; b >= 0; --b) {
    const uint32_t c = wt | (1u << b);
    if (__popcll(__ballot(tmax >= c)) >= kw) wt = c;
  }
  if (lane == 0) s_wt[wave] = wt;
  __syncthreads();
  uint32_t tau = s_wt[0];
#pragma unroll
  for (int w = 1; w < TK_THREADS / 64; ++w) tau = s_wt[w] < tau ? s_wt[w] : tau;

  auto elem_key = [&](int v, int e) -> uint32_t {
    if (BF) return (e & 1) ? (key[v][e >> 1] >> 16) : (key[v][e >> 1] & 0xFFFFu);
    return key[v][e];
  };
  auto elem_value = [&](int v, int e) -> float {
    return BF ? key16_value(elem_key(v, e)) : key32_value(elem_key(v, e));
  };
  // candidates: the logits whose raw key reaches the bound
  if (tmax >= tau) {
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        if (elem_key(v, e) >= tau) {
          const int i = s0 + (v * TK_THREADS + t) * VW + e;
          if (i < s1) {
            const int slot = atomicAdd(&s_n, 1);
            if (slot < TK_CAND) {
              s_cz[slot] = elem_value(v, e);
              s_ci[slot] = i;
            }
          }
        }
      }
  }
  __syncthreads();
  const int n = s_n;
  // every logit under the bound is at most this value
  const float below = tau == 0 ? 0.0f : (BF ? key16_value(tau - 1) : key32_value(tau - 1));
  const float below_s = scale ? below / T : below;
  uint64_t* out = a.part + ((int64_t)row * a.nseg + seg) * a.ksel;
  if (n <= TK_CAND) {
    // exact keys of the candidates, then the ksel largest by rank (keys are unique)
    for (int c = t; c < n; c += TK_THREADS) {
      float z = s_cz[c];
      if (scale) z = z / T;
      sk[c] = order_key(z, (uint32_t)s_ci[c]);
    }
    __syncthreads();
    if (n <= TK_THREADS) {
      if (t < n) {
        const uint64_t k = sk[t];
        int rank = 0;
        for (int o = 0; o < n; ++o) rank += sk[o] > k;
        if (rank < a.ksel) out[rank] = k;
        if (tau != 0 && rank == min(a.ksel, n) - 1 && !(below_s < key_value(k))) s_slow = 1;
      }
      for (int i = n + t; i < a.ksel; i += TK_THREADS) out[i] = 0;
    } else {
      const int p2 = next_pow2(n);
      for (int i = n + t; i < p2; i += TK_THREADS) sk[i] = 0;
      __syncthreads();
      bitonic_desc<TK_THREADS>(sk, p2);
      for (int i = t; i < a.ksel; i += TK_THREADS) out[i] = sk[i];
      if (t == 0 && tau != 0 && !(below_s < key_value(sk[min(a.ksel, n) - 1]))) s_slow = 1;
    }
    __syncthreads();
  } else {
    if (t == 0) s_slow = 1;
    __syncthreads();
  }
  if (s_slow) {
    // exhaustive (rare: long runs of equal logits, or a division that makes the bound tie the
    // answer): the exact ksel-th largest key by binary search over the 64-bit key space,
    // reading the segment again rather than holding every key in registers
    auto exact_key = [&](int i, bool* nan) -> uint64_t {
      float z = BF ? bf16_to_f32(((const bf16_t*)base)[rowoff + i]) : ((const float*)base)[rowoff + i];
      *nan = __builtin_isnan(z);
      if (scale) z = z / T;
      return order_key(z, (uint32_t)i);
    };
    uint64_t lo = 0, hi = ~0ull;
    while (lo < hi) {
      const uint64_t mid = lo + (hi - lo) / 2 + 1;
      if (t == 0) s_count = 0;
      __syncthreads();
      int c = 0;
      for (int i = s0 + t; i < s1; i += TK_THREADS) {
        bool nan;
        const uint64_t k = exact_key(i, &nan);
        c += (!nan && k >= mid) ? 1 : 0;
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
    for (int i = s0 + t; i < s1; i += TK_THREADS) {
      bool nan;
      const uint64_t k = exact_key(i, &nan);
      if (!nan && k >= lo) {
        const int slot = atomicAdd(&s_total, 1);
        if (slot < TK_CAND) sk[slot] = k;
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
// Merges the sorted segment lists: the largest of the segments' ksel-th keys is a bound that
// the row's ksel-th key reaches (that segment alone holds ksel keys at or above it), so only
// keys at or above it are ranked, among themselves.  Then the float32 softmax, top_p cut and
// renormalization: exponentials and divisions per lane, every running sum by one lane in the
// stated sequential order.
__global__ __launch_bounds__(FIN_THREADS) void truncate_finish_kernel(TruncArgs a, spec_probs out,
                                                                      int out_rs, float top_p,
                                                                      uint8_t* flags) {
  __shared__ uint64_t cand[FIN_SLOTS];
  __shared__ uint64_t top[SPEC_TOPK_MAX];
  __shared__ float s_p[SPEC_TOPK_MAX];
  __shared__ int s_id[SPEC_TOPK_MAX];
  __shared__ uint64_t s_theta;
  __shared__ int s_n, s_nc, s_bad, s_keep;
  __shared__ float s_S, s_Z;
  __shared__ uint8_t s_fl;
  if (a.skip && *a.skip) return;
  const int row = blockIdx.x, t = threadIdx.x, lane = t & 63;
  const int K = a.ksel, nk = a.nseg * K;
  const uint64_t* src = a.part + (int64_t)row * nk;
  // this thread's first key goes out together with wave 0's loads of the bound
  const uint64_t key0 = t < nk ? src[t] : 0;
  if (t < 64) {
    // wave 0: the bound and the bad flags
    uint64_t th = 0;
    int bad = 0;
    for (int s = lane; s < a.nseg; s += 64) {
      const uint64_t v = src[s * K + K - 1];
      th = v > th ? v : th;
      bad |= a.bad[(int64_t)row * a.nseg + s];
    }
    th = wave_max_u64(th);
    bad = __ballot(bad != 0) ? 1 : 0;
    if (t == 0) {
      s_theta = th;
      s_bad = bad;
      s_nc = 0;
    }
  }
  for (int i = t; i < K; i += FIN_THREADS) top[i] = 0;
  __syncthreads();
  const uint64_t theta = s_theta;
  for (int c = t; c < nk; c += FIN_THREADS) {
    const uint64_t key = c == t ? key0 : src[c];
    if (key != 0 && key >= theta) cand[atomicAdd(&s_nc, 1)] = key;
  }
  __syncthreads();
  const int nc = s_nc;
  for (int c = t; c < nc; c += FIN_THREADS) {
    const uint64_t key = cand[c];
    int rank = 0;
    for (int o = 0; o < nc; ++o) rank += cand[o] > key;
    if (rank < K) top[rank] = key;
  }
  __syncthreads();

  if (t < 64) {
    // entries: the leading keys that are present and finite (sorted: the rest is -inf or empty)
    bool ok = false;
    float zi = 0.0f;
    if (lane < K) {
      const uint64_t key = top[lane];
      zi = key_value(key);
      ok = key != 0 && zi != -__builtin_inff();
    }
    const uint64_t okm = __ballot(ok);
    int n = s_bad ? 0 : (~okm ? (int)__builtin_ctzll(~okm) : 64);
    const bool sampled = a.temperature > 0.0f;
    if (n > 0 && sampled && lane < n) {
      s_id[lane] = (int)key_id(top[lane]);
      s_p[lane] = expf(zi - key_value(top[0]));
    } else if (n > 0 && !sampled && lane == 0) {
      s_id[0] = (int)key_id(top[0]);
      s_p[0] = 1.0f;
    }
    if (n > 0 && !sampled) n = 1;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (n > 0 && sampled) {
      if (lane == 0) {
        float S = 0.0f;
        for (int i = 0; i < n; ++i) S = S + s_p[i];
        s_S = S;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
      if (lane < n) s_p[lane] = s_p[lane] / s_S;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
      if (lane == 0) {
        uint8_t fl = 0;
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
        s_Z = Z;
        s_keep = nkeep;
        s_fl = fl;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
      n = s_keep;
      if (lane < n) s_p[lane] = s_p[lane] / s_Z;
    } else if (lane == 0) {
      s_fl = n == 0 ? SPEC_FLAG_BAD_ROW : 0;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    if (lane == 0) {
      s_n = n;
      out.count[(int64_t)row * out_rs] = n;
      if (flags) flags[row] = s_fl;
    }
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
SPEC_DEVINL int sample_list(const int32_t* ids, const float* w, int n, float u, uint8_t* fl,
                            int* picked = nullptr) {
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
  if (picked) *picked = pick;
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

// Draft j of every sequence (one row each, rows <= 64, one wavefront) with the draft controls
// of "What is Speculative Decoding and How Does a Draft Model Work?", section "The demo, draft
// model on and off with two pairings" (the draft-probability setting): the draft model's
// confidence in a draft is the probability its list gives the drawn token; below p_min the
// sequence stops proposing before that draft.  Tokens are drawn exactly as sample_kernel draws
// them, so that the lists and tokens of the drafts kept do not depend on the controls.
__global__ __launch_bounds__(64) void sample_ctl_kernel(spec_probs lists, int list_rs, int rows, int slot,
                                                        uint64_t seed, const uint32_t* rnd_ptr, uint32_t stream_id,
                                                        int32_t* tokens, int tok_ld, DraftCtl ctl) {
  const int r = threadIdx.x;
  bool go = false;
  if (r < rows) {
    int kept = ctl.kept[r];
    int tok = 0;
    if (kept >= slot) {
      // still proposing: draw draft `slot` from its list
      const int64_t lr = (int64_t)r * list_rs;
      const int n = min(lists.count[lr], lists.cap);
      uint8_t fl = 0;
      int pick = -1;
      float conf = 0.0f;
      tok = -1;
      if (n > 0) {
        const float u = philox_uniform(seed, (uint32_t)slot, *rnd_ptr, (uint32_t)r, stream_id);
        tok = sample_list(lists.ids + lr * lists.cap, lists.probs + lr * lists.cap, n, u, &fl, &pick);
        conf = lists.probs[lr * lists.cap + pick];
      }
      if (!(conf >= ctl.p_min)) {
        // not proposed (an empty list, from logits with no finite value, stops here too)
        kept = slot - 1;
        ctl.kept[r] = kept;
        if (tok < 0) tok = 0;
      }
    }
    // a sequence that stopped before this draft gets the placeholder id 0: a valid token, so
    // that the forwards that still run over its rows (verify rows past its kept drafts, draft
    // rows while other sequences go on) stay finite; those rows are never used
    tokens[(int64_t)r * tok_ld] = tok;
    go = kept > slot;  // this sequence goes on to draft slot + 1
  }
  const uint64_t any = __ballot(go);
  if (r == 0 && any == 0) *ctl.skip = 1u;
}

__global__ void draft_ctl_init_kernel(int32_t* kept, int batch, int k, uint32_t* skip) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) kept[b] = k;
  if (b == 0) *skip = 0u;
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

// One wavefront per sequence.  The sequence's p rows (k + 1) and q rows (k) are first copied
// to LDS in one burst; lane j then tests draft j (its probabilities under p and q, its uniform
// and the ratio), the first rejected or empty row ends the run (a ballot), and lane 0 draws
// the emitted token from the residual or the bonus row with the same sequential float32 sums
// as a one-thread walk through the drafts.
__global__ __launch_bounds__(64) void accept_kernel(AcceptArgs a) {
  __shared__ int32_t s_pid[(SPEC_MAX_K + 1) * SPEC_TOPK_MAX];
  __shared__ float s_pp[(SPEC_MAX_K + 1) * SPEC_TOPK_MAX];
  __shared__ int32_t s_qid[SPEC_MAX_K * SPEC_TOPK_MAX];
  __shared__ float s_qp[SPEC_MAX_K * SPEC_TOPK_MAX];
  __shared__ float s_r[SPEC_TOPK_MAX];
  __shared__ int s_pn[SPEC_MAX_K + 1], s_qn[SPEC_MAX_K], s_am[SPEC_MAX_K + 1];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int k = a.k;
  // drafts actually proposed for this sequence (an n-gram lookup may find fewer than k);
  // the rows past them are not tested and the bonus comes from row kb
  int kb = a.kcap ? min(max(a.kcap[b], 0), k) : k;
  if (kb < a.min_draft) kb = 0;  // fewer drafts than the minimum worth checking: none
  const int32_t* d = a.drafts + (int64_t)b * k;
  int32_t* out = a.out_tok + (int64_t)b * (k + 1);
  const int pc = a.p.cap, qc = a.q.cap;
  const int64_t p0 = (int64_t)b * (k + 1), q0 = (int64_t)b * k;
  // every load of the lists first (a loop that stores each value before the next load would
  // wait one round trip per 64 entries), then the LDS stores
  constexpr int NP = SPEC_MAX_K + 1, NQ = SPEC_MAX_K;  // 64-entry rounds at most
  const int np = (k + 1) * pc, nq = a.greedy ? 0 : k * qc;
  int32_t vid[NP], wid[NQ];
  float vp[NP], wp[NQ];
#pragma unroll
  for (int r = 0; r < NP; ++r) {
    const int i = lane + 64 * r;
    if (i < np) {
      vid[r] = a.p.ids[p0 * pc + i];
      vp[r] = a.p.probs[p0 * pc + i];
    }
  }
#pragma unroll
  for (int r = 0; r < NQ; ++r) {
    const int i = lane + 64 * r;
    if (i < nq) {
      wid[r] = a.q.ids[q0 * qc + i];
      wp[r] = a.q.probs[q0 * qc + i];
    }
  }
  const int pn_l = lane <= k ? list_len(a.p, p0 + lane) : 0;
  const int qn_l = (!a.greedy && lane < k) ? list_len(a.q, q0 + lane) : 0;
#pragma unroll
  for (int r = 0; r < NP; ++r) {
    const int i = lane + 64 * r;
    if (i < np) {
      s_pid[i] = vid[r];
      s_pp[i] = vp[r];
    }
  }
#pragma unroll
  for (int r = 0; r < NQ; ++r) {
    const int i = lane + 64 * r;
    if (i < nq) {
      s_qid[i] = wid[r];
      s_qp[i] = wp[r];
    }
  }
  if (lane <= k) s_pn[lane] = pn_l;
  if (!a.greedy && lane < k) s_qn[lane] = qn_l;
  __syncthreads();

  // lane j: the test of draft j
  bool stop = false, bad = false, tie = false;
  int dj = 0;
  if (lane < kb) {
    dj = d[lane];
    const int pn = s_pn[lane];
    const int32_t* pid = s_pid + lane * pc;
    const float* pp = s_pp + lane * pc;
    if (pn <= 0) {
      // no distribution to test draft j against (its logits held no finite value): nothing
      // from j on is kept and no token is emitted (-1 signals the bad row)
      bad = stop = true;
    } else if (a.greedy) {
      const int am = list_argmax(pid, pp, pn);
      s_am[lane] = am;
      stop = dj != am;
    } else {
      const float pj = list_prob(pid, pp, pn, dj);
      const float qj = list_prob(s_qid + lane * qc, s_qp + lane * qc, s_qn[lane], dj);
      const float ratio = pj / qj;
      const float u = philox_uniform(a.seed, (uint32_t)(lane + 1), a.round, (uint32_t)b, STREAM_ACCEPT);
      tie = __builtin_isfinite(ratio) && fabsf(u - ratio) < NEAR_TIE;
      stop = !(u < ratio);
    }
  }
  const uint64_t stops = __ballot(stop), bads = __ballot(bad);
  const int n = stops ? (int)__builtin_ctzll(stops) : kb;  // drafts kept
  uint8_t fl = __ballot(tie && lane <= n) ? SPEC_FLAG_ACCEPT_TIE : 0;
  const bool bad_n = n < kb && ((bads >> n) & 1ull);
  if (lane < n) out[lane] = dj;

  // the residual max(0, p - q) over p's support of the rejecting row, one entry per lane
  const bool resid = n < kb && !bad_n && !a.greedy;
  if (resid) {
    const int pn = s_pn[n];
    if (lane < pn) {
      const int id = s_pid[n * pc + lane];
      const float qv = list_prob(s_qid + n * qc, s_qp + n * qc, s_qn[n], id);
      const float diff = s_pp[n * pc + lane] - qv;
      s_r[lane] = diff > 0.0f ? diff : 0.0f;
    }
  }
  __syncthreads();
  if (lane != 0) return;
  int emitted;
  if (n < kb) {
    if (bad_n) {
      fl |= SPEC_FLAG_BAD_ROW;
      emitted = -1;
    } else if (a.greedy) {
      emitted = s_am[n];
    } else {
      const int pn = s_pn[n];
      float Z = 0.0f;
      for (int i = 0; i < pn; ++i) Z = Z + s_r[i];
      const float ur = philox_uniform(a.seed, 0u, a.round, (uint32_t)b, STREAM_RESIDUAL);
      emitted = (Z > 0.0f) ? sample_list(s_pid + n * pc, s_r, pn, ur, &fl)
                           : sample_list(s_pid + n * pc, s_pp + n * pc, pn, ur, &fl);
    }
  } else {
    // every draft kept: bonus token from the target row after the last draft
    const int pn = s_pn[kb];
    const int32_t* pid = s_pid + kb * pc;
    const float* pp = s_pp + kb * pc;
    if (pn <= 0) {
      fl |= SPEC_FLAG_BAD_ROW;
      emitted = -1;
    } else if (a.greedy) {
      emitted = list_argmax(pid, pp, pn);
    } else {
      const float ur = philox_uniform(a.seed, 0u, a.round, (uint32_t)b, STREAM_RESIDUAL);
      emitted = sample_list(pid, pp, pn, ur, &fl);
    }
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
                           void* scratch, hipStream_t st, const uint32_t* skip) {
  TruncArgs a;
  a.skip = skip;
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

hipError_t launch_sample_ctl(const spec_probs& lists, int list_rs, int rows, int slot, uint64_t seed,
                             const uint32_t* rnd_ptr, uint32_t stream_id, int32_t* tokens, int tok_ld,
                             const DraftCtl& ctl, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (rows > 64 || !rnd_ptr || !ctl.kept || !ctl.skip) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sample_ctl_kernel, dim3(1), dim3(64), 0, st, lists, list_rs, rows, slot, seed, rnd_ptr,
                     stream_id, tokens, tok_ld, ctl);
  return hipGetLastError();
}

hipError_t launch_draft_ctl_init(int32_t* kept, int batch, int k, uint32_t* skip, hipStream_t st) {
  hipLaunchKernelGGL(draft_ctl_init_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, kept, batch, k, skip);
  return hipGetLastError();
}

hipError_t launch_accept(const AcceptArgs& a, hipStream_t st) {
  if (a.batch == 0) return hipSuccess;
  // the kernel stages a sequence's lists in LDS sized for these limits
  if (a.k < 0 || a.k > SPEC_MAX_K || a.p.cap < 1 || a.p.cap > SPEC_TOPK_MAX ||
      (!a.greedy && a.k > 0 && (a.q.cap < 1 || a.q.cap > SPEC_TOPK_MAX)))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(accept_kernel, dim3(a.batch), dim3(64), 0, st, a);
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
