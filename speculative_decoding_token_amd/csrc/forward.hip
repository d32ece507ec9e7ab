// A whole forward of a bf16 model over at most 16 token rows as one persistent launch.
//
// Launched one projection at a time, every step of a layer pays the start and drain of its
// grid, and the steps that stream little (attention, its combine) leave HBM idle.  Here one
// workgroup per compute unit (a cooperative launch, so all are resident) walks the steps of
// every layer and meets the others at grid barriers.  Before a workgroup waits at a barrier
// it already issues the first weight stages of the next projection (weights depend on
// nothing computed), so the stream keeps going across the barrier: the verify pass is one
// continuous read of the weights ("Speculative Decoding on Apple Silicon: 119% Faster...",
// section "How speculative decoding works"; "What is Speculative Decoding and How Does a
// Draft Model Work?", section "#2": one pass of the target over all drafted tokens).
//
// The projections are those of stream_core.h with their activations made coherent across
// the launch: data that one step writes and another workgroup reads in a later step
// (residual rows, their gain-multiplied float32 copy and sum-of-squares partials, q, k, new values,
// attention partials and outputs, the SwiGLU product) is stored write-through and read past
// the per-XCD L2 caches.  The attention and combine steps compute what the separate kernels
// compute, item by item (a row's result never depends on the number of rows).
//
// A barrier is a relaxed atomic arrival per workgroup after its stores have completed, a
// counter per group of workgroups, a top counter and a release word.  Every wait is bounded
// in time; once one has timed out the error word is set, every later wait ends at once and
// the launch still drains (its results are then invalid, and the error is reported to the
// host).
#include <algorithm>

#include "stream_core.h"

namespace spec {
namespace {

using namespace sk;

constexpr int SYNC_SP = 32;                          // words between barrier counters (128 bytes)
constexpr unsigned long long WAIT_TICKS = 2000000;   // 20 ms of the 100 MHz constant clock
constexpr int ATT_GROUPS = 2;                        // 4-wavefront attention groups per workgroup
constexpr int FWD_LDS_BYTES = LDS_BYTES + 64;        // + the sequences' first positions (len + pos_off)

__host__ __device__ inline int attn_group_bytes(int qt, int hd) {
  return 2 * (qt * 16 * (hd + 8) + ATTN_CHUNK * (hd + 8) + hd * (ATTN_CHUNK + 8));
}

// ---------------------------------------------------------------- grid barrier
struct Sync {
  unsigned* w;     // [8] group counters, [8] top counter, [9] release word, [10] error word
  unsigned epoch;
  unsigned long long* trace;
  int trace_cap;
};

// Every thread: wait for this wavefront's stores, meet the workgroup, arrive; `issue` runs in
// every thread before the wait (the next projection's first weight stages); leave once every
// workgroup has arrived.
template <typename F>
SPEC_DEVINL void grid_sync(Sync& s, F issue) {
  wait_vm<0>();
  wg_barrier();
  const unsigned epoch = ++s.epoch;
  const bool tr = s.trace && (int)epoch < s.trace_cap && threadIdx.x == 0;
  unsigned long long* tp = tr ? s.trace + ((size_t)epoch * gridDim.x + blockIdx.x) * 2 : nullptr;
  if (tr) tp[0] = wall_clock64();
  unsigned* rel = s.w + 9 * SYNC_SP;
  unsigned* err = s.w + 10 * SYNC_SP;
  const bool lead = threadIdx.x == 0;
  // every workgroup arrives at every barrier (the counts stay exact after a timeout); the
  // error word is read only while waiting
  if (lead) {
    const unsigned gsize = gridDim.x / 8, grp = blockIdx.x & 7;
    const unsigned a = __hip_atomic_fetch_add(s.w + grp * SYNC_SP, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a == epoch * gsize - 1) {
      const unsigned t = __hip_atomic_fetch_add(s.w + 8 * SYNC_SP, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t == epoch * 8 - 1) st<true>(rel, epoch);
    }
  }
  issue();
  if (lead) {
    const unsigned long long t0 = wall_clock64();
    while (ld<true>(rel) < epoch) {
      if (wall_clock64() - t0 > WAIT_TICKS) {
        __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      if (ld<true>(err) != 0u) break;
    }
  }
  if (tr) tp[1] = wall_clock64();
  wg_barrier();
}

// ---------------------------------------------------------------- embedding
// Workgroup m < M gathers row m: x = E[token], y = x * gain of the first norm, and the row's
// sum of squares (each thread adds its columns t, t + 512, ... in order; then a fixed sum per
// wavefront by DPP and permlane moves, and the wavefront sums in order).
SPEC_DEVINL void embed_step(const FwdArgs& a, char* sm) {
  const int m = blockIdx.x;
  if (m >= a.M) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int b = m / a.mseq, i = m % a.mseq;
  const int tok = (i == 0) ? a.first[(int64_t)b * a.first_ld] : a.rest[(int64_t)b * a.rest_ld + i - 1];
  const bool ok = tok >= 0 && tok < a.vocab;
  const bf16_t* row = (const bf16_t*)a.embed + (int64_t)(ok ? tok : 0) * a.d;
  const bf16_t* g = (const bf16_t*)a.layers[0].attn_norm;
  float sq = 0.0f;
  for (int c = t; c < a.d; c += SNW * 64) {
    const float v = ok ? bf16_to_f32(row[c]) : __builtin_nanf("");
    st<true>(a.x + (int64_t)m * a.d + c, v);
    st<true>(a.y + (int64_t)m * a.d + c, v * bf16_to_f32(g[c]));
    sq += v * v;
  }
  sq = wave_sum(sq);
  float* red = (float*)sm;
  if (lane == 0) red[wave] = sq;
  __syncthreads();
  if (t == 0) {
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < SNW; ++w) tot += red[w];
    st<true>(a.ss + (int64_t)m * a.ss_ld, tot);
  }
}

// ---------------------------------------------------------------- attention
// Item = (sequence b, kv head, chunk of 64 positions), one per 4-wavefront group, with the
// arithmetic of the stand-alone chunk kernel: scores K q^T on MFMA (lane l: query row l % 16,
// keys 4 (l / 16) + r of each 16-key tile, exactly the A-operand slots of the P V product),
// the chunk's softmax statistics in registers, P V on MFMA with V transposed in LDS.  New
// keys and values (positions L .. L + mseq - 1) come from the QKV step's rows (read past the
// L2): keys rotated, both rounded, used, and written to the cache by the group whose chunk
// holds them.
template <int HD>
struct Attn {
  static constexpr int C = ATTN_CHUNK;
  static constexpr int KP = HD + 8;
  static constexpr int VP = C + 8;
  static constexpr int HALF = HD / 2;
  static constexpr int NV = C * (HD / 8) / 256;  // 16-byte cache loads per thread and tensor

  struct Item {
    int b, kvh, chunk;
    bool ok;
  };
  static SPEC_DEVINL Item item_of(const FwdArgs& a, const int* s_len, int base) {
    const int nkv = a.cache.n_kv;
    const int items = (a.M / a.mseq) * nkv * a.nchunk;
    const int gi = threadIdx.x >> 8;
    const int it = base + blockIdx.x * ATT_GROUPS + gi;
    Item r;
    r.ok = it < items;
    const int i = r.ok ? it : 0;
    r.chunk = i % a.nchunk;
    r.kvh = (i / a.nchunk) % nkv;
    r.b = i / (a.nchunk * nkv);
    if (r.chunk * C >= s_len[r.b] + a.mseq) r.ok = false;  // past the last position
    return r;
  }
  static SPEC_DEVINL int64_t cache_base(const FwdArgs& a, int layer, const Item& it) {
    const CacheView& cv = a.cache;
    return ((((int64_t)it.b * cv.n_layers + layer) * cv.n_kv + it.kvh) * cv.cap) * HD;
  }
  // cached keys and values of the item's chunk (positions past the cache clamp to its end;
  // positions >= L are replaced after the load); nothing is read for an inactive item
  static SPEC_DEVINL void load_kv(const FwdArgs& a, int layer, const Item& it, uint4 (&kreg)[NV], uint4 (&vreg)[NV]) {
    const int t = tid_here() & 255;
    const CacheView& cv = a.cache;
    const int64_t cb = cache_base(a, layer, it);
    const uint32_t bytes = it.ok ? (uint32_t)((int64_t)cv.cap * HD * 2) : 0u;
    const __amdgpu_buffer_rsrc_t kr = rsrc((const bf16_t*)cv.k + cb, bytes);
    const __amdgpu_buffer_rsrc_t vr = rsrc((const bf16_t*)cv.v + cb, bytes);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int idx = t + 256 * v;
      const int j = idx / (HD / 8), d8 = (idx % (HD / 8)) * 8, p = it.chunk * C + j;
      const uint32_t off = (uint32_t)(min(p, cv.cap - 1) * HD + d8) * 2u;
      kreg[v] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
      vreg[v] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0));
    }
  }

  static SPEC_DEVINL void item(const FwdArgs& a, const int* s_len, int layer, char* gsm, const Item& it,
                               const uint4 (&kreg)[NV],
                               const uint4 (&vreg)[NV]) {
    const int t = tid_here() & 255, lane = t & 63, wave = t >> 6;
    const CacheView& cv = a.cache;
    const int b = it.b, kvh = it.kvh, chunk = it.chunk;
    const bool active = it.ok;
    const int mseq = a.mseq, G = a.n_q / cv.n_kv;
    const int L = s_len[b];
    const int total = L + mseq;
    const int c0 = chunk * C;
    const int R = mseq * G, QT = (R + 15) / 16;
    const int q_dim = a.n_q * HD, kv_dim = cv.n_kv * HD, qkv_ld = q_dim + 2 * kv_dim;
    bf16_t* qs = (bf16_t*)gsm;       // [QT*16][KP]
    bf16_t* ks = qs + QT * 16 * KP;  // [C][KP]
    bf16_t* vt = ks + C * KP;        // [HD][VP]
    const int64_t cb = cache_base(a, layer, it);
    bf16_t* kc = (bf16_t*)cv.k + cb;
    bf16_t* vc = (bf16_t*)cv.v + cb;
    if (active) {
      // new keys and values of this chunk (positions p0 .. p1 - 1) from the QKV step's rows:
      // the first NKH * 256 key pairs and NVH * 256 values go out with the query rows, so the
      // group waits for one round trip
      const int p0 = max(c0, L), p1 = min(c0 + C, total), nn = max(p1 - p0, 0);
      constexpr int NKH = 2, NVH = 4;
      float kx0[NKH], kx1[NKH], vx[NVH];
      float2 kcs[NKH];
      auto key_src = [&](int p) { return a.qkv + (int64_t)(b * mseq + (p - L)) * qkv_ld + q_dim + kvh * HD; };
      auto val_src = [&](int p) { return a.qkv + (int64_t)(b * mseq + (p - L)) * qkv_ld + q_dim + kv_dim + kvh * HD; };
#pragma unroll
      for (int v = 0; v < NKH; ++v) {
        const int idx = t + 256 * v;
        if (idx < nn * HALF) {
          const int p = p0 + idx / HALF, d = idx % HALF;
          kx0[v] = ld<true>(key_src(p) + d);
          kx1[v] = ld<true>(key_src(p) + d + HALF);
          kcs[v] = a.rope[(int64_t)p * HALF + d];
        }
      }
#pragma unroll
      for (int v = 0; v < NVH; ++v) {
        const int idx = t + 256 * v;
        if (idx < nn * HD) vx[v] = ld<true>(val_src(p0 + idx / HD) + idx % HD);
      }
      // query rows in batches of 8 loads per thread (one batch covers two query tiles)
      constexpr int NQB = 8;
      const int nq = (QT * 16 * HALF + 255) / 256;
      for (int v0 = 0; v0 < nq; v0 += NQB) {
        float qx0[NQB], qx1[NQB];
        float2 qcs[NQB];
#pragma unroll
        for (int v = 0; v < NQB; ++v) {
          const int idx = t + 256 * (v0 + v), d = idx % HALF;
          const int r = min(idx / HALF, R - 1);
          const int i = r / G, h = kvh * G + r % G;
          const float* src = a.qkv + (int64_t)(b * mseq + i) * qkv_ld + h * HD;
          qx0[v] = ld<true>(src + d);
          qx1[v] = ld<true>(src + d + HALF);
          qcs[v] = a.rope[(int64_t)(L + i) * HALF + d];
        }
#pragma unroll
        for (int v = 0; v < NQB; ++v) {
          const int idx = t + 256 * (v0 + v), r = idx / HALF, d = idx % HALF;
          if (r < QT * 16) {
            qs[r * KP + d] = r < R ? f32_to_bf16(qx0[v] * qcs[v].x - qx1[v] * qcs[v].y) : (bf16_t)0;
            qs[r * KP + d + HALF] = r < R ? f32_to_bf16(qx1[v] * qcs[v].x + qx0[v] * qcs[v].y) : (bf16_t)0;
          }
        }
      }
      // cached positions from the loads; positions past the end zero; new ones below
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int idx = t + 256 * v;
        const int j = idx / (HD / 8), d8 = (idx % (HD / 8)) * 8, p = c0 + j;
        if (p >= L && p < total) continue;
        const uint4 kk = p < L ? kreg[v] : make_uint4(0, 0, 0, 0);
        const uint4 vv = p < L ? vreg[v] : make_uint4(0, 0, 0, 0);
        *(uint4*)(ks + j * KP + d8) = kk;
        const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
        const int js = j ^ (((d8 >> 3) & 7) << 3);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vt[(d8 + 2 * e) * VP + js] = (bf16_t)(w[e] & 0xFFFFu);
          vt[(d8 + 2 * e + 1) * VP + js] = (bf16_t)(w[e] >> 16);
        }
      }
      // new keys: rotated, rounded, used and cached
      auto put_key = [&](int idx, float x0, float x1, float2 cs) {
        const int p = p0 + idx / HALF, d = idx % HALF, j = p - c0;
        const bf16_t lo = f32_to_bf16(x0 * cs.x - x1 * cs.y);
        const bf16_t hi = f32_to_bf16(x1 * cs.x + x0 * cs.y);
        ks[j * KP + d] = lo;
        ks[j * KP + d + HALF] = hi;
        kc[(int64_t)p * HD + d] = lo;
        kc[(int64_t)p * HD + d + HALF] = hi;
      };
#pragma unroll
      for (int v = 0; v < NKH; ++v)
        if (t + 256 * v < nn * HALF) put_key(t + 256 * v, kx0[v], kx1[v], kcs[v]);
      for (int idx = t + 256 * NKH; idx < nn * HALF; idx += 256) {
        const int p = p0 + idx / HALF, d = idx % HALF;
        put_key(idx, ld<true>(key_src(p) + d), ld<true>(key_src(p) + d + HALF), a.rope[(int64_t)p * HALF + d]);
      }
      // new values: rounded, used (transposed, in the swizzled V^T layout) and cached
      auto put_val = [&](int idx, float x) {
        const int p = p0 + idx / HD, d = idx % HD, j = p - c0;
        const bf16_t v16 = f32_to_bf16(x);
        vt[d * VP + (j ^ (((d >> 3) & 7) << 3))] = v16;
        vc[(int64_t)p * HD + d] = v16;
      };
#pragma unroll
      for (int v = 0; v < NVH; ++v)
        if (t + 256 * v < nn * HD) put_val(t + 256 * v, vx[v]);
      for (int idx = t + 256 * NVH; idx < nn * HD; idx += 256) put_val(idx, ld<true>(val_src(p0 + idx / HD) + idx % HD));
    }
    __syncthreads();
    if (active) {
      const int n = lane & 15, g = lane >> 4;
      constexpr int DT = HD / 16;
      const int wpt = min(QT == 1 ? 4 : (QT == 2 ? 2 : 1), DT);
      const int part = wave % wpt;
      const int dts = DT / wpt;
      for (int qt = wave / wpt; qt < QT; qt += 4 / wpt) {
        f32x4_t s[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int stp = 0; stp < HD / 32; ++stp) {
            const uint4 av = *(const uint4*)(ks + (kt * 16 + n) * KP + stp * 32 + 8 * g);
            const uint4 bv = *(const uint4*)(qs + (qt * 16 + n) * KP + stp * 32 + 8 * g);
            s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                            __builtin_bit_cast(bf16x8_t, bv), s[kt], 0, 0, 0);
          }
        }
        const int r = qt * 16 + n;
        const int pos = (r < R) ? L + r / G : -1;
        float mx = -__builtin_inff();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int p = c0 + kt * 16 + 4 * g + rr;
            const float v = (p <= pos) ? s[kt][rr] * a.scale : -__builtin_inff();
            s[kt][rr] = v;
            mx = fmaxf(mx, v);
          }
        mx = xor32_max(xor16_max(mx));
        bf16x8_t pa[2][2];
        const float l = p_operands(s, mx, pa);
        int rowoff[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r2 = qt * 16 + 4 * g + rr;
          rowoff[rr] = -1;
          if (r2 < R) {
            const int i2 = r2 / G, h2 = kvh * G + r2 % G;
            rowoff[rr] = (((b * mseq + i2) * a.n_q + h2) * a.nchunk + chunk) * (HD + 2);
          }
        }
        for (int dt = part * dts; dt < (part + 1) * dts; ++dt) {
          f32x4_t o = f32x4_t{0.f, 0.f, 0.f, 0.f};
          const int dim = dt * 16 + n;
          const int swz = ((dim >> 3) & 7) << 3;
#pragma unroll
          for (int stp = 0; stp < 2; ++stp) {
            const bf16_t* vrow = vt + dim * VP;
            const uint2 x0 = *(const uint2*)(vrow + ((stp * 32 + 4 * g) ^ swz));
            const uint2 x1 = *(const uint2*)(vrow + ((stp * 32 + 16 + 4 * g) ^ swz));
            const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, make_uint4(x0.x, x0.y, x1.x, x1.y));
            o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[stp][0], vb, o, 0, 0, 0);
            o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[stp][1], vb, o, 0, 0, 0);
          }
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (rowoff[rr] >= 0) st<true>(a.part + rowoff[rr] + dim, o[rr]);
        }
        if (part == 0 && g == 0 && r < R) {
          const int i = r / G, h = kvh * G + r % G;
          float* P = a.part + ((int64_t)((b * mseq + i) * a.n_q + h) * a.nchunk + chunk) * (HD + 2);
          st<true>(P + HD, mx);
          st<true>(P + HD + 1, l);
        }
      }
    }
    __syncthreads();
  }
};

// The cached keys and values of a group's first item (positions before the new tokens, which
// the QKV step does not touch) are loaded while the workgroup waits at the barrier before the
// attention step: their round trip overlaps the barrier's.
template <int HD>
SPEC_DEVINL void attn_prefetch(const FwdArgs& a, const int* s_len, int layer, uint4 (&kreg)[Attn<HD>::NV],
                               uint4 (&vreg)[Attn<HD>::NV]) {
  Attn<HD>::load_kv(a, layer, Attn<HD>::item_of(a, s_len, 0), kreg, vreg);
}

template <int HD>
SPEC_DEVINL void attn_step(const FwdArgs& a, const int* s_len, int layer, char* sm, uint4 (&kreg)[Attn<HD>::NV],
                           uint4 (&vreg)[Attn<HD>::NV]) {
  using A = Attn<HD>;
  const int nkv = a.cache.n_kv;
  const int items = (a.M / a.mseq) * nkv * a.nchunk;
  const int G = a.n_q / nkv, QT = (a.mseq * G + 15) / 16;
  const int gi = threadIdx.x >> 8;
  char* gsm = sm + gi * attn_group_bytes(QT, HD);
  const int slots = gridDim.x * ATT_GROUPS;
  for (int base = 0; base < items; base += slots) {
    const typename A::Item it = A::item_of(a, s_len, base);
    if (base > 0) A::load_kv(a, layer, it, kreg, vreg);  // the first item's came with the barrier
    A::item(a, s_len, layer, gsm, it, kreg, vreg);
  }
}

// ---------------------------------------------------------------- combine
// Unit = (row m, q head h), one per 256-thread half of the workgroup: the chunk maxima and
// weights exp(m_c - max) from one wavefront, the weighted value sums with the chunks split
// over 256 / head_dim thread groups, added back in a fixed order.  Each thread's values go
// out before the weights are known (coherent loads in a loop would wait for one another).
template <int HD>
SPEC_DEVINL void combine_step(const FwdArgs& a, const int* s_len, char* red) {
  const int txc = tid_here(), half = txc >> 8, t = txc & 255;
  float* s_w = (float*)red + half * (ATTN_MAX_CHUNKS + 257);
  float* s_part = s_w + ATTN_MAX_CHUNKS;
  float* s_den = s_part + 256;
  const int units = a.M * a.n_q;
  for (int base = 0; base < units; base += gridDim.x * 2) {
    const int u = base + blockIdx.x * 2 + half;
    const bool ok = u < units;
    const int uu = ok ? u : 0;
    const int m = uu / a.n_q, h = uu % a.n_q;
    const int b = m / a.mseq, i = m % a.mseq;
    const int pos = s_len[b] + i;
    const int nch = pos / ATTN_CHUNK + 1;
    const float* P = a.part + (int64_t)uu * a.nchunk * (HD + 2);
    constexpr int GROUPS = 256 / HD;
    constexpr int NR = 8;  // chunk values per thread loaded before the weights
    const int g = t / HD, d = t % HD;
    // coherent plain loads (not atomics), so that unrolled runs of them are all in flight
    const __amdgpu_buffer_rsrc_t pr = rsrc(P, (uint32_t)(a.nchunk * (HD + 2) * 4));
    auto pval = [&](int c) {
      return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, (uint32_t)(c * (HD + 2) + d) * 4u, 0,
                                                                           CPOL_SC1));
    };
    float pv[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int c = g + GROUPS * q;
      pv[q] = c < nch ? pval(c) : 0.0f;
    }
    if (t < 64) {
      constexpr int PER = ATTN_MAX_CHUNKS / 64;
      float mc[PER], lc[PER];
      float mx = -__builtin_inff();
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int c = t + 64 * q;
        mc[q] = c < nch ? ld<true>(P + c * (HD + 2) + HD) : -__builtin_inff();
        lc[q] = c < nch ? ld<true>(P + c * (HD + 2) + HD + 1) : 0.0f;
        mx = fmaxf(mx, mc[q]);
      }
      mx = wave_max(mx);
      float den = 0.0f;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int c = t + 64 * q;
        if (c < nch) {
          const float w = expf(mc[q] - mx);
          s_w[c] = w;
          den += lc[q] * w;
        }
      }
      den = wave_sum(den);
      if (t == 0) *s_den = den;
    }
    __syncthreads();
    float o = 0.0f;
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int c = g + GROUPS * q;
      if (c < nch) o += pv[q] * s_w[c];
    }
#pragma unroll 8
    for (int c = g + GROUPS * NR; c < nch; c += GROUPS) o += pval(c) * s_w[c];
    s_part[t] = o;
    __syncthreads();
    if (ok && t < HD) {
      float tot = 0.0f;
#pragma unroll
      for (int q = 0; q < GROUPS; ++q) tot += s_part[q * HD + t];
      st<true>((bf16_t*)a.attn + (int64_t)m * a.n_q * HD + h * HD + t, f32_to_bf16(tot / *s_den));
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- projections of a layer
SPEC_DEVINL StreamArgs qkv_args(const FwdArgs& a, int l) {
  const spec_layer_weights& w = a.layers[l];
  StreamArgs g{};
  g.w0 = w.wq;
  g.w1 = w.wk;
  g.w2 = w.wv;
  g.rows0 = a.q_dim;
  g.rows1 = a.kv_dim;
  g.rows2 = a.kv_dim;
  g.K = a.d;
  g.nunits = (a.q_dim + 2 * a.kv_dim) / 16;
  g.x = a.y;
  g.ss_in = a.ss;
  g.np_in = l == 0 ? 1 : a.d / 16;
  g.ss_ld = a.ss_ld;
  g.eps = a.eps;
  g.M = a.M;
  g.out = a.qkv;
  g.ld = a.q_dim + 2 * a.kv_dim;
  return g;
}
SPEC_DEVINL StreamArgs o_args(const FwdArgs& a, int l) {
  StreamArgs g{};
  g.w0 = a.layers[l].wo;
  g.rows0 = a.d;
  g.K = a.q_dim;
  g.nunits = a.d / 16;
  g.x = a.attn;
  g.M = a.M;
  g.out = a.x;
  g.ld = a.d;
  g.ss_out = a.ss;
  g.ss_ld = a.ss_ld;
  g.y_out = a.y;
  g.y_gain = a.layers[l].ffn_norm;
  return g;
}
SPEC_DEVINL StreamArgs gu_args(const FwdArgs& a, int l) {
  StreamArgs g{};
  g.w0 = a.layers[l].wg;
  g.w1 = a.layers[l].wu;
  g.rows0 = a.ffn;
  g.K = a.d;
  g.nunits = a.ffn / 16;
  g.x = a.y;
  g.ss_in = a.ss;
  g.np_in = a.d / 16;
  g.ss_ld = a.ss_ld;
  g.eps = a.eps;
  g.M = a.M;
  g.h = a.h;
  return g;
}
SPEC_DEVINL StreamArgs down_args(const FwdArgs& a, int l) {
  StreamArgs g{};
  g.w0 = a.layers[l].wd;
  g.rows0 = a.d;
  g.K = a.ffn;
  g.nunits = a.d / 16;
  g.x = a.h;
  g.M = a.M;
  g.out = a.x;
  g.ld = a.d;
  g.ss_out = a.ss;
  g.ss_ld = a.ss_ld;
  g.y_out = a.y;
  g.y_gain = l + 1 < a.n_layers ? a.layers[l + 1].attn_norm : a.final_norm;
  return g;
}
SPEC_DEVINL StreamArgs head_args(const FwdArgs& a) {
  StreamArgs g{};
  g.w0 = a.lm_head;
  g.rows0 = a.vocab;
  g.K = a.d;
  g.nunits = a.vocab / 16;
  g.x = a.y;
  g.ss_in = a.ss;
  g.np_in = a.d / 16;
  g.ss_ld = a.ss_ld;
  g.eps = a.eps;
  g.M = a.M;
  g.out = a.logits;
  g.ld = a.vocab;
  return g;
}

// ---------------------------------------------------------------- the forward
// NSTD: stages of a reduction over d (d / 1024), NSTQ: over the attention width (q_dim / 1024).
template <int NSTD, int NSTQ, int HD>
__global__ __launch_bounds__(SNW * 64) void forward_kernel(FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  if (a.skip && *a.skip) return;  // every workgroup leaves before the first barrier
  using QKV = Gemm<EPI_QKV_ROWS, NSTD, true>;
  using OP = Gemm<EPI_RESID, NSTQ, true>;
  using GU = Gemm<EPI_SWIGLU, 2 * NSTD, true>;
  using DN = Gemm<EPI_RESID, 0, true>;
  using HEAD = Gemm<EPI_STORE, NSTD, true>;
  constexpr int P = RING - 1;  // weight stages issued ahead of a barrier
  Sync s{a.sync, 0u, a.trace, a.trace_cap};
  if (a.trace && threadIdx.x == 0 && a.trace_cap > 0) a.trace[(size_t)blockIdx.x * 2] = wall_clock64();
  uint4 kreg[Attn<HD>::NV], vreg[Attn<HD>::NV];
  char* red = sm + RING * STAGE;  // the combine step's LDS, clear of the ring
  // first position of each sequence, read once
  int* s_len = (int*)(sm + LDS_BYTES);
  if (threadIdx.x < (unsigned)(a.M / a.mseq)) s_len[threadIdx.x] = a.len[threadIdx.x] + a.pos_off;
  __syncthreads();
  embed_step(a, sm);
  grid_sync(s, [&] { QKV::prefetch(qkv_args(a, 0), sm, P); });
#pragma clang loop unroll(disable)
  for (int l = 0; l < a.n_layers; ++l) {
    QKV::run(qkv_args(a, l), sm, P);
    grid_sync(s, [&] { attn_prefetch<HD>(a, s_len, l, kreg, vreg); });
    attn_step<HD>(a, s_len, l, sm, kreg, vreg);
    grid_sync(s, [&] { OP::prefetch(o_args(a, l), sm, P); });
    combine_step<HD>(a, s_len, red);
    grid_sync(s, [] {});
    OP::run(o_args(a, l), sm, P);
    grid_sync(s, [&] { GU::prefetch(gu_args(a, l), sm, P); });
    GU::run(gu_args(a, l), sm, P);
    grid_sync(s, [&] { DN::prefetch(down_args(a, l), sm, P); });
    DN::run(down_args(a, l), sm, P);
    if (l + 1 < a.n_layers) grid_sync(s, [&] { QKV::prefetch(qkv_args(a, l + 1), sm, P); });
    else if (a.logits) grid_sync(s, [&] { HEAD::prefetch(head_args(a), sm, P); });
  }
  if (a.logits) HEAD::run(head_args(a), sm, P);
}

// Counters and the release word start at zero in every launch; the error word is sticky (a
// timed-out barrier leaves the context's results invalid until it is recreated).
__global__ void sync_reset_kernel(unsigned* w) {
  const int i = threadIdx.x;
  if (i < 10) w[i * SYNC_SP] = 0u;
}

template <int NSTD, int NSTQ, int HD>
const void* fwd_ptr() {
  return (const void*)forward_kernel<NSTD, NSTQ, HD>;
}

const void* fwd_select(int d, int q_dim, int hd) {
  if (hd != 128) return nullptr;
  const int nd = d / 1024, nq = q_dim / 1024;
  if (d % 1024 || q_dim % 1024) return nullptr;
  if (nd == 1 && nq == 1) return fwd_ptr<1, 1, 128>();
  if (nd == 1 && nq == 2) return fwd_ptr<1, 2, 128>();
  if (nd == 2 && nq == 2) return fwd_ptr<2, 2, 128>();
  // (d = 5120 is left to the per-launch schedules: its one-launch kernel does not fit the
  // register file without spilling)
  if (nd == 4 && nq == 4) return fwd_ptr<4, 4, 128>();
  return nullptr;
}

}  // namespace

bool forward_supported(int M, int mseq, int d, int n_q, int n_kv, int hd, int ffn, int vocab) {
  if (M < 1 || M > 16 || mseq < 1 || M % mseq) return false;
  if (!fwd_select(d, n_q * hd, hd)) return false;
  const int G = n_q / n_kv, QT = (mseq * G + 15) / 16;
  if (QT > 6 || ATT_GROUPS * attn_group_bytes(QT, hd) > RING * STAGE) return false;
  if (ffn % 1024 || vocab % 16 || (n_q * hd + 2 * n_kv * hd) % 16) return false;
  return true;
}

size_t forward_sync_bytes(int batch, int n_kv) {
  (void)batch;
  (void)n_kv;
  return 11 * SYNC_SP * 4;
}

hipError_t forward_init(int* grid) {
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const void* ks[] = {fwd_ptr<1, 1, 128>(), fwd_ptr<1, 2, 128>(), fwd_ptr<2, 2, 128>(), fwd_ptr<4, 4, 128>()};
  int fit = 1 << 30;
  for (const void* k : ks) {
    e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, FWD_LDS_BYTES);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k, SNW * 64, FWD_LDS_BYTES);
    if (e != hipSuccess) return e;
    fit = std::min(fit, nb);
  }
  // one workgroup per compute unit, a multiple of 8 (the barrier's groups)
  *grid = fit >= 1 ? ncu / 8 * 8 : 0;
  return hipSuccess;
}

hipError_t launch_forward(const FwdArgs& a, int grid, hipStream_t st) {
  const void* k = fwd_select(a.d, a.q_dim, a.cache.hd);
  if (!k || grid < 8 || grid % 8 || a.M > grid) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sync_reset_kernel, dim3(1), dim3(64), 0, st, a.sync);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  FwdArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchCooperativeKernel(k, dim3(grid), dim3(SNW * 64), args, (unsigned)FWD_LDS_BYTES, st);
}

}  // namespace spec
