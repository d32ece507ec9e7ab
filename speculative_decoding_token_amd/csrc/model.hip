// Decoder kernels of the verify pass: embedding gather, RMSNorm, the skinny projections,
// block-causal attention against the cache, and the small state kernels.
//
// A verify is one target forward over the last accepted token and the K drafts
// ("What is Speculative Decoding and How Does a Draft Model Work?", section "#2": the target
// checks all drafted tokens in a single pass, the way it reads a prompt).  At M = K+1 rows
// the pass streams every weight once, so it is bound by HBM bandwidth, not by arithmetic
// ("Speculative Decoding on Apple Silicon: 119% Faster...", section "How speculative
// decoding works": most of a pass moves weights rather than computing on them).
//
// Every kernel computes a row's result with the same arithmetic in the same order whatever
// the number of rows M, so row i of a K+1-row verify is bit-identical to a one-row forward
// of the same token at the same position.
#include <algorithm>

#include "kernels.h"

namespace spec {

// ---------------------------------------------------------------- RoPE table
// cos/sin of pos * theta^(-2i/head_dim), evaluated in double and stored as float.
__global__ void rope_table_kernel(float2* table, int cap, int hd, double theta) {
  const int half = hd / 2;
  const int64_t n = (int64_t)cap * half;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int pos = (int)(idx / half), i = (int)(idx % half);
    const double inv = pow(theta, -2.0 * (double)i / (double)hd);
    const double ang = (double)pos * inv;
    table[idx] = make_float2((float)cos(ang), (float)sin(ang));
  }
}

// ---------------------------------------------------------------- embedding gather
// Row m = (seq b, i): token first[b*first_ld] for i == 0, else rest[b*rest_ld + i-1].  Also
// leaves the row's sum of squares in ss[m * ss_ld] (fixed reduction order) for the RMSNorm of
// the first projection and, when y is set (bf16), row * gain in float32: that projection's
// input before its 1/rms.
template <int DT>
__global__ __launch_bounds__(256) void embed_kernel(const void* E, int d, int vocab,
                                                    const int32_t* first, int first_ld,
                                                    const int32_t* rest, int rest_ld, int mseq,
                                                    float* x, float* ss, int ss_ld, float* y,
                                                    const bf16_t* gain) {
  using A = Act<DT>;
  constexpr int NT = 256, NV = 16;  // threads; elements a thread loads before its first store
  __shared__ float red[NT];
  const int m = blockIdx.x, b = m / mseq, i = m % mseq, t = threadIdx.x;
  const int tok = (i == 0) ? first[(int64_t)b * first_ld] : rest[(int64_t)b * rest_ld + i - 1];
  const bool ok = tok >= 0 && tok < vocab;
  const typename A::T* row = (const typename A::T*)E + (int64_t)(ok ? tok : 0) * d;
  const bool gy = DT == SPEC_DTYPE_BF16 && y;
  // without y the gain loads read the row's own first bytes, unused
  const bf16_t* gp = gy ? gain : (const bf16_t*)row;
  // Thread t takes elements t, t + NT, ...: all NV loads of a group (embedding and gain, at
  // clamped indices, with no branch or arithmetic between them) go out before its stores, so
  // a row of up to NT * NV elements waits for one round trip after the token id, not one per
  // element group.
  float sq = 0.0f;
  for (int c0 = 0; c0 < d; c0 += NT * NV) {
    typename A::T v[NV];
    bf16_t g[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int c = min(c0 + t + NT * q, d - 1);
      v[q] = row[c];
      g[q] = gp[c];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load of the group ahead of the stores
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int c = c0 + t + NT * q;
      if (c < d) {
        const float val = ok ? A::load(v, q) : __builtin_nanf("");
        x[(int64_t)m * d + c] = val;
        if (gy) y[(int64_t)m * d + c] = val * bf16_to_f32(g[q]);
        sq += val * val;
      }
    }
  }
  red[t] = sq;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  if (ss && t == 0) ss[(int64_t)m * ss_ld] = red[0];

}

// ---------------------------------------------------------------- MTP input
// The multi-token-prediction layer reads the target's hidden state h at position t-1 and
// the embedding of the token at t, each RMS-normalized with its own gain, side by side
// ("What is Speculative Decoding and How Does a Draft Model Work?", section "MTP and the
// other drafting methods": extra layers predicting the following tokens; "Speculative
// decoding on Apple Silicon" (OptiQ docs), section "Serving and the Lab": a projection
// followed by a final layer).  One workgroup per row; both sums of squares in one pass.
template <int DT>
__global__ __launch_bounds__(256) void mtp_input_kernel(MtpInArgs a) {
  using A = Act<DT>;
  typedef typename A::T T;
  __shared__ float red[2][256];
  const int m = blockIdx.x, b = m / a.R, i = m % a.R, t = threadIdx.x, d = a.d;
  const float* h = a.h + b * a.h_ss + i * a.h_rs;
  const int tok = a.tok[(int64_t)b * a.tok_ld + (a.tok_pos ? a.tok_pos[b] : 0) + i];
  const bool ok = tok >= 0 && tok < a.vocab;
  const T* e = (const T*)a.embed + (int64_t)(ok ? tok : 0) * d;
  const T* gh = (const T*)a.norm_h;
  const T* ge = (const T*)a.norm_e;
  // Thread t takes elements t, t + NT, ...; the loads of a group of NV of them (both rows and,
  // when the whole row is one group, both gains) go out together, ahead of any arithmetic.
  constexpr int NT = 256, NV = 16;
  const bool one = d <= NT * NV;  // then the values stay in registers for the second pass
  float hv[NV];
  T ev[NV], ghv[NV], gev[NV];
  float sh = 0.0f, se = 0.0f;
  for (int c0 = 0; c0 < d; c0 += NT * NV) {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int c = min(c0 + t + NT * q, d - 1);
      hv[q] = h[c];
      ev[q] = e[c];
      if (one) {
        ghv[q] = gh[c];
        gev[q] = ge[c];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < NV; ++q)
      if (c0 + t + NT * q < d) {
        const float x = hv[q], y = A::load(ev, q);
        sh += x * x;
        se += y * y;
      }
  }
  red[0][t] = sh;
  red[1][t] = se;
  __syncthreads();
  for (int s2 = 128; s2 > 0; s2 >>= 1) {
    if (t < s2) {
      red[0][t] += red[0][t + s2];
      red[1][t] += red[1][t + s2];
    }
    __syncthreads();
  }
  const float ih = 1.0f / sqrtf(red[0][0] / (float)d + a.eps);
  const float ie = ok ? 1.0f / sqrtf(red[1][0] / (float)d + a.eps) : __builtin_nanf("");
  T* o = (T*)a.out + (int64_t)m * 2 * d;
  for (int c0 = 0; c0 < d; c0 += NT * NV) {
    if (!one) {
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        const int c = min(c0 + t + NT * q, d - 1);
        hv[q] = h[c];
        ev[q] = e[c];
        ghv[q] = gh[c];
        gev[q] = ge[c];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int c = c0 + t + NT * q;
      if (c < d) {
        A::store(o, c, hv[q] * ih * A::load(ghv, q));
        A::store(o, d + c, A::load(ev, q) * ie * A::load(gev, q));
      }
    }
  }
}

__global__ void gather_last_kernel(const float* x, const float* ss, int ss_ld, int d, int R, const int32_t* len,
                                   const int32_t* mlen, float* x1, float* ss1) {
  const int b = blockIdx.x, t = threadIdx.x;
  const int r = mlen ? min(max(len[b] - mlen[b], 0), R - 1) : 0;
  const float* src = x + ((int64_t)b * R + r) * d;
  for (int c = t; c < d; c += blockDim.x) x1[(int64_t)b * d + c] = src[c];
  if (ss)
    for (int c = t; c < ss_ld; c += blockDim.x) ss1[(int64_t)b * ss_ld + c] = ss[((int64_t)b * R + r) * ss_ld + c];
}

__global__ void copy_rows_f32_kernel(const float* src, int64_t src_ss, int R, int d, float* dst, int64_t dst_ss) {
  const int row = blockIdx.x, b = row / R, i = row % R;
  for (int c = threadIdx.x; c < d; c += blockDim.x)
    dst[b * dst_ss + (int64_t)i * d + c] = src[b * src_ss + (int64_t)i * d + c];
}

__global__ void len_from_kernel(int32_t* dst, const int32_t* src, int batch, int add) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) dst[b] = src[b] + add;
}

// ---------------------------------------------------------------- RMSNorm
// y = x / sqrt(mean(x^2) + eps) * g, rounded to the model dtype.  Fixed reduction order.
template <int DT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* x, const void* g, float eps,
                                                      int d, void* y) {
  using A = Act<DT>;
  __shared__ float red[256];
  const int m = blockIdx.x, t = threadIdx.x;
  const float* xr = x + (int64_t)m * d;
  float ss = 0.0f;
  for (int c = t; c < d; c += 256) ss += xr[c] * xr[c];
  red[t] = ss;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  const float inv = 1.0f / sqrtf(red[0] / (float)d + eps);
  const typename A::T* gg = (const typename A::T*)g;
  typename A::T* yr = (typename A::T*)y + (int64_t)m * d;
  for (int c = t; c < d; c += 256) A::store(yr, c, xr[c] * inv * A::load(gg, c));
}

// ---------------------------------------------------------------- projection epilogues
SPEC_DEVINL float silu(float g) { return g / (1.0f + expf(-g)); }

template <int DT, int EPI>
SPEC_DEVINL void gemm_epilogue(const GemmArgs& a, int mat, int m, int n, float v0, float v1) {
  using A = Act<DT>;
  if (EPI == EPI_STORE) {
    a.out[(int64_t)m * a.ld + n] = v0;
  } else if (EPI == EPI_RESID) {
    a.out[(int64_t)m * a.ld + n] += v0;
  } else if (EPI == EPI_SWIGLU) {
    A::store((typename A::T*)a.h, (int64_t)m * a.rows[0] + n, silu(v0) * v1);
  } else {  // EPI_QKV
    if (mat == 0) {
      a.q_stage[(int64_t)m * a.rows[0] + n] = v0;
    } else if (mat == 1) {
      a.k_stage[(int64_t)m * a.rows[1] + n] = v0;
    } else {
      const CacheView& c = a.cache;
      const int b = m / a.rm.mseq;
      const int pos = a.rm.len[b] + a.rm.pos_off + m % a.rm.mseq;
      const int kvh = n / c.hd, dd = n % c.hd;
      const int64_t idx = ((((int64_t)b * c.n_layers + a.layer) * c.n_kv + kvh) * c.cap + pos) * c.hd + dd;
      A::store((typename A::T*)c.v, idx, v0);
    }
  }
}

// ---------------------------------------------------------------- bf16 projection (MFMA)
// out[m, n] = sum_k W[n, k] * x[m, k] for M <= 16*NT token rows.
//
// One workgroup owns 16 weight rows (two 16-row tiles, gate and up, for SwiGLU) over the
// whole K; its 8 wavefronts split K by interleaved 32-wide steps and meet in LDS, so no
// partial sum leaves the workgroup.  Each step is one v_mfma_f32_16x16x32_bf16 per tile:
// A = 16 weight rows x 32 k (lane l loads 16 bytes of row l%16 at k offset 8*(l/16)),
// B = 32 k x 16 token rows (the same k slice of x, zero for rows >= M).  The MFMA's 16x
// padding of the token dimension costs nothing here: the pass is bound by streaming W.
//
// With NORM the input is RMSNorm(x) * g with no pass of its own: the producer of the residual
// x left the float32 rows x * g and the rows' sum-of-squares partials, the block adds the
// partials into 1/sqrt(mean(x^2) + eps) before its main loop (their loads go out with the
// first weights) and rounds (x * g) times it to bf16 as it loads each input slice.  A residual
// epilogue leaves, per block, the sum of squares of its 16 updated columns of each row and,
// when asked, those columns times the next norm's gain in float32.
SPEC_DEVINL uint32_t pack_bf16x2(float lo, float hi) { return bf16x2_pack(lo, hi); }

// y[m, k] = x[m, k] * gain[k] in float32: a projection's RMSNorm input rows when the producer
// of x left none.
__global__ __launch_bounds__(256) void gain_rows_kernel(const float* x, const bf16_t* gain, int K, float* y) {
  const int m = blockIdx.x;
  for (int k = threadIdx.x; k < K; k += 256) y[(int64_t)m * K + k] = x[(int64_t)m * K + k] * bf16_to_f32(gain[k]);
}

// Single-tile instances of 16 wavefronts are held to 64 VGPRs: two workgroups per compute
// unit, so 384 or 512 tiles (QKV, output and down projections) run in one round.
template <int EPI, int NT, bool NORM, int GEMM_NW>
__global__ __launch_bounds__(GEMM_NW * 64, (GEMM_NW == 16 && EPI != EPI_SWIGLU) ? 8 : 1) void gemm_bf16_kernel(
    GemmArgs a) {
  // k-steps per load group: 8 KB of weights in flight per wave and tile either way (halved for
  // several token tiles of float32 RMSNorm inputs, whose slices take twice the registers)
  constexpr int GEMM_U = ((GEMM_NW == 16 || NT == 4) ? 4 : 8) / ((NORM && NT >= 2) ? 2 : 1);
  constexpr int TILES = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int PSS = TILES == 2 ? 4 : 2;  // partials per lane loaded ahead (a row's first 64 * PSS)
  __shared__ f32x4_t red[GEMM_NW][TILES][NT][64];
  __shared__ float s_inv[16 * NT];
  __shared__ float s_sq[16 * NT][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int mat = 0, r0 = blockIdx.x * 16;
  if (EPI == EPI_QKV) {
    if (r0 >= a.rows[0]) {
      r0 -= a.rows[0];
      mat = 1;
      if (r0 >= a.rows[1]) {
        r0 -= a.rows[1];
        mat = 2;
      }
    }
  }
  const int K = a.K, nsteps = K >> 5, M = a.rm.M;
  const int koff = 8 * (lane >> 4);
  // row `wave`'s partials lane, lane + 64, ... (zero past the count: adding them changes nothing)
  float pss[PSS];
  if (NORM) {
#pragma unroll
    for (int q = 0; q < PSS; ++q) {
      const int p = lane + 64 * q;
      pss[q] = (wave < M && p < a.np_in) ? a.ss_in[(int64_t)wave * a.ss_ld + p] : 0.0f;
    }
  }
  const bf16_t* wp[TILES];
  wp[0] = (const bf16_t*)a.w[mat] + (int64_t)(r0 + (lane & 15)) * K + koff;
  if (TILES == 2) wp[TILES - 1] = (const bf16_t*)a.w[1] + (int64_t)(r0 + (lane & 15)) * K + koff;
  bool xv[NT];
  int64_t xrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int m = nt * 16 + (lane & 15);
    xv[nt] = m < M;
    xrow[nt] = (int64_t)(xv[nt] ? m : 0) * K + koff;
  }
  // first group of weights in flight before anything else
  uint4 wa[TILES][GEMM_U];
#pragma unroll
  for (int u = 0; u < GEMM_U; ++u) {
    const int s = wave + u * GEMM_NW;
#pragma unroll
    for (int t = 0; t < TILES; ++t)
      wa[t][u] = s < nsteps ? *(const uint4*)(wp[t] + (int64_t)s * 32) : make_uint4(0, 0, 0, 0);
  }

  f32x4_t acc[TILES][NT];
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[t][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // RMSNorm input: 1/rms of each row (lane j adds the row's partials j, j + 64, ... in order,
  // then a fixed xor butterfly; wave w takes rows w, w + GEMM_NW, ...), then per token tile
  // the factor of this lane's row
  float rv[NT];
  if (NORM) {
    for (int r = wave; r < M; r += GEMM_NW) {
      float sum = 0.0f;
      int p0 = lane;
      if (r == wave) {
#pragma unroll
        for (int q = 0; q < PSS; ++q) sum += pss[q];
        p0 = lane + 64 * PSS;
      }
      for (int p = p0; p < a.np_in; p += 64) sum += a.ss_in[(int64_t)r * a.ss_ld + p];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
      if (lane == 0) s_inv[r] = 1.0f / sqrtf(sum / (float)K + a.eps);
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) rv[nt] = xv[nt] ? s_inv[nt * 16 + (lane & 15)] : 0.0f;
  }

  for (int s0 = wave; s0 < nsteps; s0 += GEMM_NW * GEMM_U) {
    uint4 xb[NT][GEMM_U];
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u) {
      const int s = s0 + u * GEMM_NW;
      const bool ok = s < nsteps;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (NORM) {
          const float* xp = (const float*)a.x + xrow[nt] + (int64_t)s * 32;
          const uint4 lo = (ok && xv[nt]) ? *(const uint4*)xp : make_uint4(0, 0, 0, 0);
          const uint4 hi = (ok && xv[nt]) ? *(const uint4*)(xp + 4) : make_uint4(0, 0, 0, 0);
          const float r = rv[nt];
          xb[nt][u] = make_uint4(pack_bf16x2(__uint_as_float(lo.x) * r, __uint_as_float(lo.y) * r),
                                 pack_bf16x2(__uint_as_float(lo.z) * r, __uint_as_float(lo.w) * r),
                                 pack_bf16x2(__uint_as_float(hi.x) * r, __uint_as_float(hi.y) * r),
                                 pack_bf16x2(__uint_as_float(hi.z) * r, __uint_as_float(hi.w) * r));
        } else {
          xb[nt][u] = (ok && xv[nt]) ? *(const uint4*)((const bf16_t*)a.x + xrow[nt] + (int64_t)s * 32)
                                     : make_uint4(0, 0, 0, 0);
        }
      }
    }
    // next group of weights while this one is multiplied
    uint4 wn[TILES][GEMM_U];
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u) {
      const int s = s0 + (GEMM_U + u) * GEMM_NW;
#pragma unroll
      for (int t = 0; t < TILES; ++t)
        wn[t][u] = s < nsteps ? *(const uint4*)(wp[t] + (int64_t)s * 32) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u)
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, wa[t][u]), __builtin_bit_cast(bf16x8_t, xb[nt][u]),
              acc[t][nt], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u)
#pragma unroll
      for (int t = 0; t < TILES; ++t) wa[t][u] = wn[t][u];
  }
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) red[wave][t][nt][lane] = acc[t][nt];
  __syncthreads();

  // D layout of the 16x16 MFMA: lane l holds column l%16 (token), rows 4*(l/16)+r (weight row)
  for (int e = threadIdx.x; e < NT * 256; e += GEMM_NW * 64) {
    const int nt = e >> 8, l = (e >> 2) & 63, r = e & 3;
    const int m = nt * 16 + (l & 15);
    const int n = r0 + 4 * (l >> 4) + r;
    if (m < M) {
      float v[TILES];
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < GEMM_NW; ++w) s += red[w][t][nt][l][r];
        v[t] = s;
      }
      if (EPI == EPI_RESID) {
        const float xn = a.out[(int64_t)m * a.ld + n] + v[0];
        a.out[(int64_t)m * a.ld + n] = xn;
        s_sq[m][n - r0] = xn * xn;
        if (a.y_out) ((float*)a.y_out)[(int64_t)m * a.ld + n] = xn * bf16_to_f32(((const bf16_t*)a.y_gain)[n]);
      } else {
        gemm_epilogue<SPEC_DTYPE_BF16, EPI>(a, mat, m, n, v[0], v[TILES - 1]);
      }
    }
  }
  if (EPI == EPI_RESID && a.ss_out) {
    __syncthreads();
    const int m = threadIdx.x;
    if (m < M && m < 16 * NT) {
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) ss += s_sq[m][j];
      a.ss_out[(int64_t)m * a.ss_ld + blockIdx.x] = ss;
    }
  }
}

// ---------------------------------------------------------------- f32 projection (VALU)
// One wavefront per output row, lanes over k, a fixed xor-butterfly reduction.
constexpr int GF_MAXM = 32;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int TILES = (EPI == EPI_SWIGLU) ? 2 : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int total = a.rows[0];
  if (EPI == EPI_QKV) total += a.rows[1] + a.rows[2];
  int r = blockIdx.x * 4 + wave;
  if (r >= total) return;
  int mat = 0;
  if (EPI == EPI_QKV) {
    if (r >= a.rows[0]) {
      r -= a.rows[0];
      mat = 1;
      if (r >= a.rows[1]) {
        r -= a.rows[1];
        mat = 2;
      }
    }
  }
  const int K = a.K, M = a.rm.M;
  const float* w0 = (const float*)a.w[mat] + (int64_t)r * K;
  const float* w1 = (const float*)a.w[TILES == 2 ? 1 : mat] + (int64_t)r * K;
  const float* x = (const float*)a.x;
  float acc[TILES][GF_MAXM];
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int m = 0; m < GF_MAXM; ++m) acc[t][m] = 0.0f;
  for (int k = lane; k < K; k += 64) {
    const float a0 = w0[k];
    const float a1 = TILES == 2 ? w1[k] : 0.0f;
#pragma unroll
    for (int m = 0; m < GF_MAXM; ++m) {
      if (m < M) {
        const float xv = x[(int64_t)m * K + k];
        acc[0][m] += a0 * xv;
        if (TILES == 2) acc[TILES - 1][m] += a1 * xv;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int m = 0; m < GF_MAXM; ++m) {
      if (m < M) {
        float v = acc[t][m];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        acc[t][m] = v;
      }
    }
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < GF_MAXM; ++m)
      if (m < M) gemm_epilogue<SPEC_DTYPE_F32, EPI>(a, mat, m, r, acc[0][m], acc[TILES - 1][m]);
  }
}

// ---------------------------------------------------------------- attention
// Split-context attention of the K+1 query rows against the cache.  Workgroup = (chunk of
// 64 positions, kv head, sequence); it serves every q head of the kv head's group and every
// query row.  Query row i sits at position L+i and sees keys 0..L+i: the causal mask inside
// the drafted block.  New keys (positions L..L+M-1) are rotated here, used, and written to
// the cache by the one workgroup whose chunk holds them.  Each workgroup leaves, per query
// row and head, the chunk's (max, sum of exp, weighted value sum); attn_combine merges the
// chunks in order.  Chunks are fixed ranges of absolute positions, so a row's result does
// not depend on how many rows the pass has.
// A sequence length read as a vector load (the address passed through a VGPR), to be issued
// before the loads that do not depend on it: vector loads complete in order, so waiting for
// this one leaves those in flight, where a scalar load would be waited for together with the
// kernel arguments before anything else is issued.
SPEC_DEVINL int len_first(const int32_t* p) {
  uint64_t v = (uint64_t)p;
  asm volatile("" : "+v"(v));
  return *(const __attribute__((address_space(1))) int32_t*)v;  // global, not flat
}

template <int DT>
__global__ __launch_bounds__(256) void attn_chunk_kernel(AttnArgs a) {
  if (a.skip && *a.skip) return;
  using A = Act<DT>;
  typedef typename A::T T;
  extern __shared__ float sm[];
  constexpr int C = ATTN_CHUNK;
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const CacheView& cv = a.cache;
  const int hd = cv.hd, half = hd / 2, mseq = a.rm.mseq, G = a.n_q / cv.n_kv;
  const int L = a.rm.len[b] + a.rm.pos_off;
  const int total = L + mseq;
  const int c0 = chunk * C;
  if (c0 >= total) return;
  const int R = mseq * G;
  const int q_dim = a.n_q * hd, kv_dim = cv.n_kv * hd;
  float* qs = sm;                  // [R][hd]
  float* ks = qs + R * hd;         // [C][hd+1]
  float* vs = ks + C * (hd + 1);   // [C][hd]
  float* ss = vs + C * hd;         // [R][C]
  float* ml = ss + R * C;          // [R][2]

  for (int idx = t; idx < R * half; idx += 256) {
    const int r = idx / half, d = idx % half;
    const int i = r / G, h = kvh * G + r % G;
    const int pos = L + i;
    const float* src = a.q_stage + (int64_t)(b * mseq + i) * q_dim + h * hd;
    const float x0 = src[d], x1 = src[d + half];
    const float2 cs = a.rope[(int64_t)pos * half + d];
    qs[r * hd + d] = A::round(x0 * cs.x - x1 * cs.y);
    qs[r * hd + d + half] = A::round(x1 * cs.x + x0 * cs.y);
  }
  const int64_t cbase = ((((int64_t)b * cv.n_layers + a.layer) * cv.n_kv + kvh) * cv.cap) * hd;
  T* kc = (T*)cv.k + cbase;
  const T* vc = (const T*)cv.v + cbase;
  for (int idx = t; idx < C * half; idx += 256) {
    const int j = idx / half, d = idx % half, p = c0 + j;
    float k0 = 0.0f, k1 = 0.0f;
    if (p < L) {
      k0 = A::load(kc, (int64_t)p * hd + d);
      k1 = A::load(kc, (int64_t)p * hd + d + half);
    } else if (p < total) {
      const float* src = a.k_stage + (int64_t)(b * mseq + (p - L)) * kv_dim + kvh * hd;
      const float x0 = src[d], x1 = src[d + half];
      const float2 cs = a.rope[(int64_t)p * half + d];
      k0 = A::round(x0 * cs.x - x1 * cs.y);
      k1 = A::round(x1 * cs.x + x0 * cs.y);
      A::store(kc, (int64_t)p * hd + d, k0);
      A::store(kc, (int64_t)p * hd + d + half, k1);
    }
    ks[j * (hd + 1) + d] = k0;
    ks[j * (hd + 1) + d + half] = k1;
  }
  for (int idx = t; idx < C * hd; idx += 256) {
    const int j = idx / hd, d = idx % hd, p = c0 + j;
    vs[j * hd + d] = p < total ? A::load(vc, (int64_t)p * hd + d) : 0.0f;
  }
  __syncthreads();

  // scores: thread = (key j, row group); rows r = group + 4q
  {
    const int j = t & 63, rg = t >> 6;
    constexpr int RQ = ATTN_ROWS_MAX / 4;
    float acc[RQ];
#pragma unroll
    for (int q = 0; q < RQ; ++q) acc[q] = 0.0f;
    for (int d = 0; d < hd; ++d) {
      const float kd = ks[j * (hd + 1) + d];
#pragma unroll
      for (int q = 0; q < RQ; ++q) {
        const int r = rg + 4 * q;
        if (r < R) acc[q] += qs[r * hd + d] * kd;
      }
    }
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int r = rg + 4 * q;
      if (r < R) {
        const int pos = L + r / G, p = c0 + j;
        ss[r * C + j] = (p <= pos) ? acc[q] * a.scale : -__builtin_inff();
      }
    }
  }
  __syncthreads();

  // softmax pieces per row: a wavefront per row, a lane per key
  {
    const int lane = t & 63, w = t >> 6;
    for (int r = w; r < R; r += 4) {
      const float s = ss[r * C + lane];
      float mx = s;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const float e = (mx == -__builtin_inff() || s == -__builtin_inff()) ? 0.0f : expf(s - mx);
      float l = e;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
      ss[r * C + lane] = e;
      if (lane == 0) {
        ml[2 * r] = mx;
        ml[2 * r + 1] = l;
      }
    }
  }
  __syncthreads();

  // weighted values: thread = (dim d, row group)
  {
    const int groups = 256 / hd;
    const int d = t % hd, rg = t / hd;
    constexpr int RO = ATTN_ROWS_MAX / 2;
    float o[RO];
#pragma unroll
    for (int q = 0; q < RO; ++q) o[q] = 0.0f;
    for (int j = 0; j < C; ++j) {
      const float v = vs[j * hd + d];
#pragma unroll
      for (int q = 0; q < RO; ++q) {
        const int r = rg + groups * q;
        if (r < R) o[q] += ss[r * C + j] * v;
      }
    }
#pragma unroll
    for (int q = 0; q < RO; ++q) {
      const int r = rg + groups * q;
      if (r < R) {
        const int i = r / G, h = kvh * G + r % G;
        const int m = b * mseq + i;
        float* P = a.part + ((int64_t)(m * a.n_q + h) * a.nchunk + chunk) * (hd + 2);
        P[d] = o[q];
        if (d == 0) {
          P[hd] = ml[2 * r];
          P[hd + 1] = ml[2 * r + 1];
        }
      }
    }
  }
}

// bf16 version on MFMA.  Scores S^T = K Q^T come out of v_mfma_f32_16x16x32_bf16 with lane
// l holding query row l%16 and keys 4*(l/16)+r of each 16-key tile; those are exactly the
// A-operand slots of the following P V product for two key tiles at once (with the key
// order inside a 32-key step permuted the same way on the V side), so P never leaves the
// registers.  V is staged transposed in LDS so that each lane's 8 keys are two 8-byte
// reads.  P = exp(s - m) stays float32 up to the product: it enters the MFMA as the sum of
// two bf16 operands (hi = bf16(P), lo = bf16(P - hi), 16 significant bits together, a
// relative error below 2^-16), and the row sum adds the float32 values.
template <int HD, int QTM>
__global__ __launch_bounds__(256) void attn_chunk_mfma_kernel(AttnArgs a) {
  constexpr int C = ATTN_CHUNK;  // 64 keys
  constexpr int KP = HD + 8;     // LDS pitch of q and K rows (bf16 elements)
  constexpr int VP = C + 8;      // LDS pitch of V^T rows
  constexpr int HALF = HD / 2;
  extern __shared__ __attribute__((aligned(16))) char smraw[];
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const CacheView& cv = a.cache;
  const int mseq = a.rm.mseq, G = a.n_q / cv.n_kv;
  const int c0 = chunk * C;
  const int R = mseq * G, QT = (R + 15) / 16;
  const int q_dim = a.n_q * HD, kv_dim = cv.n_kv * HD;
  const int L = len_first(a.rm.len + b) + a.rm.pos_off;
  bf16_t* qs = (bf16_t*)smraw;   // [QT*16][KP]
  bf16_t* ks = qs + QT * 16 * KP;  // [C][KP]
  bf16_t* vt = ks + C * KP;        // [HD][VP]

  const int64_t cbase = ((((int64_t)b * cv.n_layers + a.layer) * cv.n_kv + kvh) * cv.cap) * HD;
  bf16_t* kc = (bf16_t*)cv.k + cbase;
  const bf16_t* vc = (const bf16_t*)cv.v + cbase;
  // cached keys and values, 16 bytes at a time, go out right behind the length (no address
  // depends on it), so the two round trips overlap; zeros past the end are put in after the
  // loads
  constexpr int NV = C * (HD / 8) / 256;
  uint4 kreg[NV], vreg[NV];
  // branch-free: addresses are clamped into the cache, out-of-range values zeroed after the load
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int idx = t + 256 * v;
    const int j = idx / (HD / 8), d8 = (idx % (HD / 8)) * 8, p = c0 + j;
    const int pc = min(p, cv.cap - 1);
    kreg[v] = *(const uint4*)(kc + (int64_t)pc * HD + d8);
    vreg[v] = *(const uint4*)(vc + (int64_t)pc * HD + d8);
  }
  const int total = L + mseq;
  // (a chunk past the last position runs through with every key masked; no combine reads it)
  // the new keys of this chunk (positions p0 .. p1-1): the first NKH * 256 of their
  // (position, pair) items are loaded here too, so the block waits for one round trip
  const int p0 = max(c0, L), p1 = min(c0 + C, total), nnew = max(p1 - p0, 0) * HALF;
  constexpr int NKH = 2;
  float kx0[NKH], kx1[NKH];
  float2 kcs[NKH];
#pragma unroll
  for (int v = 0; v < NKH; ++v) {
    const int idx = t + 256 * v;
    if (idx < nnew) {
      const int p = p0 + idx / HALF, d = idx % HALF;
      const float* src = a.k_stage + (int64_t)(b * mseq + (p - L)) * kv_dim + kvh * HD;
      kx0[v] = src[d];
      kx1[v] = src[d + HALF];
      kcs[v] = a.rope[(int64_t)p * HALF + d];
    }
  }

  // a skipped draft launch leaves here, its argument fetched with the others
  if (a.skip && *a.skip) return;
  // query rows: every load of the thread first (ATTN_ROWS_MAX*HALF/256 slots), then the rotation
  {
    constexpr int NQ = (QTM * 16 * HALF + 255) / 256;  // QTM: most query tiles this instance serves
    float qx0[NQ], qx1[NQ];
    float2 qcs[NQ];
#pragma unroll
    for (int v = 0; v < NQ; ++v) {
      const int idx = t + 256 * v, d = idx % HALF;
      const int r = min(idx / HALF, R - 1);  // clamped: rows >= R are zeroed below
      const int i = r / G, h = kvh * G + r % G;
      const float* src = a.q_stage + (int64_t)(b * mseq + i) * q_dim + h * HD;
      qx0[v] = src[d];
      qx1[v] = src[d + HALF];
      qcs[v] = a.rope[(int64_t)(L + i) * HALF + d];
    }
#pragma unroll
    for (int v = 0; v < NQ; ++v) {
      const int idx = t + 256 * v, r = idx / HALF, d = idx % HALF;
      if (r < QT * 16) {
        qs[r * KP + d] = r < R ? f32_to_bf16(qx0[v] * qcs[v].x - qx1[v] * qcs[v].y) : (bf16_t)0;
        qs[r * KP + d + HALF] = r < R ? f32_to_bf16(qx1[v] * qcs[v].x + qx0[v] * qcs[v].y) : (bf16_t)0;
      }
    }
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int idx = t + 256 * v;
    const int j = idx / (HD / 8), d8 = (idx % (HD / 8)) * 8, p = c0 + j;
    // value selects (a select of the two sources' addresses would put kreg in scratch memory)
    const uint4 kz = make_uint4(0, 0, 0, 0);
    const uint4 kk = p < L ? kreg[v] : kz;
    if (p < L || p >= total) *(uint4*)(ks + j * KP + d8) = kk;
    const uint4 vv = p < total ? vreg[v] : kz;
    const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
    // V^T rows d8..d8+7 are all in swizzle group d8/8: the key index is xor-ed with 8*(group&7),
    // which spreads the 16 lanes that write one key over 8 banks and keeps 8-key runs whole
    const int js = j ^ (((d8 >> 3) & 7) << 3);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vt[(d8 + 2 * e) * VP + js] = (bf16_t)(w[e] & 0xFFFFu);
      vt[(d8 + 2 * e + 1) * VP + js] = (bf16_t)(w[e] >> 16);
    }
  }
  // new keys in this chunk: rotate, round, use, and write to the cache
  {
    auto put = [&](int idx, float x0, float x1, float2 cs) {
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
      if (t + 256 * v < nnew) put(t + 256 * v, kx0[v], kx1[v], kcs[v]);
    for (int idx = t + 256 * NKH; idx < nnew; idx += 256) {
      const int p = p0 + idx / HALF, d = idx % HALF;
      const float* src = a.k_stage + (int64_t)(b * mseq + (p - L)) * kv_dim + kvh * HD;
      put(idx, src[d], src[d + HALF], a.rope[(int64_t)p * HALF + d]);
    }
  }
  __syncthreads();

  const int n = lane & 15, g = lane >> 4;
  // waves per query tile: 4 for one tile, 2 for two, else 1; each recomputes the tile's
  // scores (16 MFMAs) and takes its share of the HD/16 output dim tiles
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
      for (int st = 0; st < HD / 32; ++st) {
        const uint4 av = *(const uint4*)(ks + (kt * 16 + n) * KP + st * 32 + 8 * g);
        const uint4 bv = *(const uint4*)(qs + (qt * 16 + n) * KP + st * 32 + 8 * g);
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                        __builtin_bit_cast(bf16x8_t, bv), s[kt], 0, 0, 0);
      }
    }
    // lane holds query row r = qt*16 + n, keys c0 + kt*16 + 4g + rr
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
    bf16x8_t pa[2][2];  // P = hi + lo, two bf16 operands per 32-key step
    const float l = p_operands(s, mx, pa);
    // this lane's rows of the output tile: 4g + rr
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
      for (int st = 0; st < 2; ++st) {
        const bf16_t* vr = vt + dim * VP;
        const uint2 x0 = *(const uint2*)(vr + ((st * 32 + 4 * g) ^ swz));
        const uint2 x1 = *(const uint2*)(vr + ((st * 32 + 16 + 4 * g) ^ swz));
        const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, make_uint4(x0.x, x0.y, x1.x, x1.y));
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[st][0], vb, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[st][1], vb, o, 0, 0, 0);
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        if (rowoff[rr] >= 0) a.part[rowoff[rr] + dim] = o[rr];
    }
    if (part == 0 && g == 0 && r < R) {
      const int i = r / G, h = kvh * G + r % G;
      float* P = a.part + ((int64_t)((b * mseq + i) * a.n_q + h) * a.nchunk + chunk) * (HD + 2);
      P[HD] = mx;
      P[HD + 1] = l;
    }
  }
}

// The same chunk for few query rows (R <= ATTN_FEW_ROWS, head_dim 128: a draft model at one or
// two rows) on the vector ALUs, where 16-row MFMA tiles would be mostly padding.  The cached
// keys and values stay in the registers they are loaded into: thread t holds rows
// j = t / 16 + 16 v (v < 4) of the chunk, dims 8 (t % 16) .. + 7.  Only the query rows and the
// chunk's new keys (rotated here) pass through LDS.  Scores: each thread's 8-dim products in
// order, then summed over the 16 threads of a row by a fixed butterfly; the chunk softmax per
// row in float32 (maximum over the chunk, then exp(s - max)); P V: each thread's products over
// its four keys, summed over the four rows of threads of a wavefront and then over the four
// wavefronts in order.  Partials in the layout the combine kernel reads.
__global__ __launch_bounds__(256) void attn_chunk_few_kernel(AttnArgs a) {
  constexpr int HD = 128, C = ATTN_CHUNK, KP = HD + 8, HALF = HD / 2;
  constexpr int RM = ATTN_FEW_ROWS;
  constexpr int NV = C * (HD / 8) / 256;  // key rows a thread holds
  static_assert(NV == 4, "four key rows a thread: one per row of 16 threads of a wavefront");
  __shared__ __attribute__((aligned(16))) bf16_t ks[C * KP];  // the new keys' rows only
  __shared__ __attribute__((aligned(16))) float qf[RM][HD];
  __shared__ __attribute__((aligned(16))) float opart[4][RM][HD];
  __shared__ float wred[2][4][RM];
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const CacheView& cv = a.cache;
  const int mseq = a.rm.mseq, G = a.n_q / cv.n_kv;
  const int L = a.rm.len[b] + a.rm.pos_off;
  const int total = L + mseq;
  const int c0 = chunk * C;
  if (c0 >= total) return;
  const int R = mseq * G;
  const int kv_dim = cv.n_kv * HD, q_dim = a.n_q * HD;
  const int64_t cbase = ((((int64_t)b * cv.n_layers + a.layer) * cv.n_kv + kvh) * cv.cap) * HD;
  bf16_t* kc = (bf16_t*)cv.k + cbase;
  const bf16_t* vc = (const bf16_t*)cv.v + cbase;
  // every load first: cached K and V rows of the chunk (16 threads per 256-byte row), the
  // query pair of this thread, and the first new-key pairs
  const int d8 = (t & 15) * 8;
  uint4 kreg[NV], vreg[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int j = (t >> 4) + 16 * v;
    const int pc = min(c0 + j, cv.cap - 1);
    kreg[v] = *(const uint4*)(kc + (int64_t)pc * HD + d8);
    vreg[v] = *(const uint4*)(vc + (int64_t)pc * HD + d8);
  }
  const int qr = t / HALF, qd = t % HALF;  // query row and rotation pair of this thread
  float qx0 = 0.f, qx1 = 0.f;
  float2 qcs = make_float2(0.f, 0.f);
  if (qr < R) {
    const int i = qr / G, h = kvh * G + qr % G;
    const float* src = a.q_stage + (int64_t)(b * mseq + i) * q_dim + h * HD;
    qx0 = src[qd];
    qx1 = src[qd + HALF];
    qcs = a.rope[(int64_t)(L + i) * HALF + qd];
  }
  const int p0 = max(c0, L), p1 = min(c0 + C, total), nnew = max(p1 - p0, 0) * HALF;
  constexpr int NKH = 2;
  float kx0[NKH], kx1[NKH];
  float2 kcs[NKH];
#pragma unroll
  for (int v = 0; v < NKH; ++v) {
    const int idx = t + 256 * v;
    if (idx < nnew) {
      const int p = p0 + idx / HALF, d = idx % HALF;
      const float* src = a.k_stage + (int64_t)(b * mseq + (p - L)) * kv_dim + kvh * HD;
      kx0[v] = src[d];
      kx1[v] = src[d + HALF];
      kcs[v] = a.rope[(int64_t)p * HALF + d];
    }
  }
  // a skipped draft launch leaves here, its argument fetched with the others
  if (a.skip && *a.skip) return;
  // staging: q rotated and rounded as the MFMA kernel does; the new keys rotated, rounded and
  // written to LDS and to the cache
  if (qr < RM) {
    qf[qr][qd] = qr < R ? bf16_to_f32(f32_to_bf16(qx0 * qcs.x - qx1 * qcs.y)) : 0.0f;
    qf[qr][qd + HALF] = qr < R ? bf16_to_f32(f32_to_bf16(qx1 * qcs.x + qx0 * qcs.y)) : 0.0f;
  }
  {
    auto put = [&](int idx, float x0, float x1, float2 cs) {
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
      if (t + 256 * v < nnew) put(t + 256 * v, kx0[v], kx1[v], kcs[v]);
    for (int idx = t + 256 * NKH; idx < nnew; idx += 256) {
      const int p = p0 + idx / HALF, d = idx % HALF;
      const float* src = a.k_stage + (int64_t)(b * mseq + (p - L)) * kv_dim + kvh * HD;
      put(idx, src[d], src[d + HALF], a.rope[(int64_t)p * HALF + d]);
    }
  }
  __syncthreads();

  // this thread's keys: cached ones as loaded, new ones from LDS, none past the end (their
  // values zero, so that a stale row never meets a zero weight)
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int j = (t >> 4) + 16 * v, p = c0 + j;
    if (p >= L && p < total) kreg[v] = *(const uint4*)(ks + j * KP + d8);
    if (p >= total) vreg[v] = make_uint4(0, 0, 0, 0);
  }
  float kf[NV][8];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const uint32_t kw[4] = {kreg[v].x, kreg[v].y, kreg[v].z, kreg[v].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kf[v][2 * e] = __uint_as_float(kw[e] << 16);
      kf[v][2 * e + 1] = __uint_as_float(kw[e] & 0xFFFF0000u);
    }
  }
  // scores, masked and scaled; the chunk maximum of each row over this thread's four keys, the
  // four rows of threads of the wavefront and the four wavefronts
  float s[NV][RM], mx[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    mx[r] = -__builtin_inff();
    if (r < R) {
      const float4 q0 = *(const float4*)(&qf[r][d8]);
      const float4 q1 = *(const float4*)(&qf[r][d8 + 4]);
      const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += kf[v][e] * qv[e];
        acc = row16_sum(acc);
        const int p = c0 + (t >> 4) + 16 * v;
        s[v][r] = p <= L + r / G ? acc * a.scale : -__builtin_inff();
        mx[r] = fmaxf(mx[r], s[v][r]);
      }
      mx[r] = xor32_max(xor16_max(mx[r]));
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RM; ++r) wred[0][wave][r] = mx[r];
  }
  __syncthreads();
  // weights exp(s - max) in float32; P V over this thread's keys in order and the weight sums,
  // then over the wavefront's four rows of threads
  float o[RM][8], lsum[RM];
  float vf[NV][8];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const uint32_t vw[4] = {vreg[v].x, vreg[v].y, vreg[v].z, vreg[v].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vf[v][2 * e] = __uint_as_float(vw[e] << 16);
      vf[v][2 * e + 1] = __uint_as_float(vw[e] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    lsum[r] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[r][e] = 0.0f;
    if (r < R) {
      const float m = fmaxf(fmaxf(wred[0][0][r], wred[0][1][r]), fmaxf(wred[0][2][r], wred[0][3][r]));
      mx[r] = m;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const float w = (m == -__builtin_inff() || s[v][r] == -__builtin_inff()) ? 0.0f : expf(s[v][r] - m);
        lsum[r] += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[r][e] += w * vf[v][e];
      }
      lsum[r] = xor32_sum(xor16_sum(lsum[r]));
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] = xor32_sum(xor16_sum(o[r][e]));
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < RM; ++r)
      if (r < R) {
        *(float4*)(&opart[wave][r][d8]) = make_float4(o[r][0], o[r][1], o[r][2], o[r][3]);
        *(float4*)(&opart[wave][r][d8 + 4]) = make_float4(o[r][4], o[r][5], o[r][6], o[r][7]);
      }
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RM; ++r) wred[1][wave][r] = lsum[r];
  }
  __syncthreads();
  // the four wavefronts' partials added in order: thread t takes (row, dim) pairs t, t + 256
  for (int idx = t; idx < R * HD; idx += 256) {
    const int r = idx / HD, d = idx % HD;
    const int i = r / G, h = kvh * G + r % G;
    float* P = a.part + ((int64_t)((b * mseq + i) * a.n_q + h) * a.nchunk + chunk) * (HD + 2);
    P[d] = ((opart[0][r][d] + opart[1][r][d]) + opart[2][r][d]) + opart[3][r][d];
    if (d == 0) {
      P[HD] = fmaxf(fmaxf(wred[0][0][r], wred[0][1][r]), fmaxf(wred[0][2][r], wred[0][3][r]));
      P[HD + 1] = ((wred[1][0][r] + wred[1][1][r]) + wred[1][2][r]) + wred[1][3][r];
    }
  }
}

// Merges the chunks of one (row, head): weights exp(m_c - max) from one wavefront (every
// chunk statistic loaded at once), then the weighted value sums with the chunks split over
// 256/head_dim thread groups and added back in a fixed order.  Each thread's first values
// are loaded before the weights are computed, so the merge waits for about one round trip.
template <int DT>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  using A = Act<DT>;
  constexpr int NR = 32;  // chunk values per thread held in registers (the rest are loaded later)
  __shared__ float s_w[ATTN_MAX_CHUNKS];
  __shared__ float s_part[256];
  __shared__ float s_den;
  const int row = blockIdx.x, t = threadIdx.x;
  const int hd = a.cache.hd;
  const int m = row / a.n_q, h = row % a.n_q;
  const int b = m / a.rm.mseq, i = m % a.rm.mseq;
  const int pos = a.rm.len[b] + a.rm.pos_off + i;
  const int nch = pos / ATTN_CHUNK + 1;
  const float* P = a.part + (int64_t)row * a.nchunk * (hd + 2);
  const int groups = 256 / hd, g = t / hd, d = t % hd;
  // this thread's values (chunks g, g + groups, ...) go out before the weights are known
  float pv[NR];
#pragma unroll
  for (int q = 0; q < NR; ++q) {
    const int c = g + groups * q;
    pv[q] = c < nch ? P[c * (hd + 2) + d] : 0.0f;
  }
  if (a.skip && *a.skip) return;  // a skipped draft launch (argument fetched with the others)
  if (t < 64) {
    constexpr int PER = ATTN_MAX_CHUNKS / 64;
    float mc[PER], lc[PER];
    float mx = -__builtin_inff();
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int c = t + 64 * q;
      mc[q] = c < nch ? P[c * (hd + 2) + hd] : -__builtin_inff();
      lc[q] = c < nch ? P[c * (hd + 2) + hd + 1] : 0.0f;
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
    if (t == 0) s_den = den;
  }
  __syncthreads();
  float o = 0.0f;
#pragma unroll
  for (int q = 0; q < NR; ++q) {
    const int c = g + groups * q;
    if (c < nch) o += pv[q] * s_w[c];
  }
  for (int c = g + groups * NR; c < nch; c += groups) o += P[c * (hd + 2) + d] * s_w[c];
  s_part[t] = o;
  __syncthreads();
  if (t < hd) {
    float tot = 0.0f;
    for (int q = 0; q < groups; ++q) tot += s_part[q * hd + t];
    A::store((typename A::T*)a.out, (int64_t)m * a.n_q * hd + h * hd + t, tot / s_den);
  }
}

// ---------------------------------------------------------------- small state kernels
__global__ void fill_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
__global__ void copy_i32_kernel(const int32_t* s, int s_ld, int32_t* d, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) d[i] = s[(int64_t)i * s_ld];
}
template <typename T>
__global__ void kv_load_kernel(const T* k, const T* v, CacheView c, int seq, int length) {
  const int64_t n = (int64_t)c.n_layers * c.n_kv * length * c.hd;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int dd = (int)(idx % c.hd);
    int64_t r = idx / c.hd;
    const int p = (int)(r % length);
    r /= length;  // r = layer * n_kv + kvh
    const int64_t dst = (((int64_t)seq * c.n_layers * c.n_kv + r) * c.cap + p) * c.hd + dd;
    ((T*)c.k)[dst] = k[idx];
    ((T*)c.v)[dst] = v[idx];
  }
}
__global__ void set_len_kernel(int32_t* len, int seq, int value) { len[seq] = value; }
__global__ void add_len_kernel(int32_t* len, int batch, int delta) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) len[b] += delta;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_rope_table(float2* table, int cap, int hd, float theta, hipStream_t st) {
  const int64_t n = (int64_t)cap * (hd / 2);
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, st, table, cap, hd, (double)theta);
  return hipGetLastError();
}

hipError_t launch_embed(int dtype, const void* E, int d, int vocab, const int32_t* first,
                        int first_ld, const int32_t* rest, int rest_ld, int M, int mseq, float* x,
                        float* ss, int ss_ld, void* y, const void* gain, hipStream_t st) {
  if (dtype == SPEC_DTYPE_BF16)
    hipLaunchKernelGGL(embed_kernel<SPEC_DTYPE_BF16>, dim3(M), dim3(256), 0, st, E, d, vocab, first,
                       first_ld, rest, rest_ld, mseq, x, ss, ss_ld, (float*)y, (const bf16_t*)gain);
  else
    hipLaunchKernelGGL(embed_kernel<SPEC_DTYPE_F32>, dim3(M), dim3(256), 0, st, E, d, vocab, first,
                       first_ld, rest, rest_ld, mseq, x, ss, ss_ld, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_mtp_input(int dtype, const MtpInArgs& a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  if (dtype == SPEC_DTYPE_BF16)
    hipLaunchKernelGGL(mtp_input_kernel<SPEC_DTYPE_BF16>, dim3(a.M), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(mtp_input_kernel<SPEC_DTYPE_F32>, dim3(a.M), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gather_last(const float* x, const float* ss, int ss_ld, int d, int R, const int32_t* len,
                              const int32_t* mlen, int batch, float* x1, float* ss1, hipStream_t st) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_last_kernel, dim3(batch), dim3(256), 0, st, x, ss, ss_ld, d, R, len, mlen, x1, ss1);
  return hipGetLastError();
}

hipError_t launch_copy_rows_f32(const float* src, int64_t src_ss, int R, int d, int batch, float* dst,
                                int64_t dst_ss, hipStream_t st) {
  if (batch * R == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_rows_f32_kernel, dim3(batch * R), dim3(256), 0, st, src, src_ss, R, d, dst, dst_ss);
  return hipGetLastError();
}

hipError_t launch_len_from(int32_t* dst, const int32_t* src, int batch, int add, hipStream_t st) {
  hipLaunchKernelGGL(len_from_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, dst, src, batch, add);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int dtype, const float* x, const void* g, float eps, int M, int d, void* y,
                          hipStream_t st) {
  if (dtype == SPEC_DTYPE_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<SPEC_DTYPE_BF16>, dim3(M), dim3(256), 0, st, x, g, eps, d, y);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<SPEC_DTYPE_F32>, dim3(M), dim3(256), 0, st, x, g, eps, d, y);
  return hipGetLastError();
}

// 16 wavefronts per workgroup when there are few 16-row tiles (each wave then has one group
// of loads in flight for K = 4096), 8 for the LM head's thousands of tiles.
template <int EPI, bool NORM, int NW>
static hipError_t gemm_bf16_nw(const GemmArgs& a, int blocks, hipStream_t st) {
  const int M = a.rm.M;
  if (M <= 16)
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI, 1, NORM, NW>), dim3(blocks), dim3(NW * 64), 0, st, a);
  else if (M <= 32)
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI, 2, NORM, NW>), dim3(blocks), dim3(NW * 64), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI, 4, NORM, 8>), dim3(blocks), dim3(8 * 64), 0, st, a);
  return hipGetLastError();
}

template <int EPI, bool NORM>
static hipError_t gemm_bf16_nt(const GemmArgs& a, int blocks, hipStream_t st) {
  return blocks <= 1024 ? gemm_bf16_nw<EPI, NORM, 16>(a, blocks, st) : gemm_bf16_nw<EPI, NORM, 8>(a, blocks, st);
}

hipError_t launch_gain_rows(const float* x, const void* gain, int M, int K, void* y, hipStream_t st) {
  if (M == 0) return hipSuccess;
  if (K % 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gain_rows_kernel, dim3(M), dim3(256), 0, st, x, (const bf16_t*)gain, K, (float*)y);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t st) {
  int rows = a.rows[0];
  if (epi == EPI_QKV) rows += a.rows[1] + a.rows[2];
  if (a.rm.M == 0 || rows == 0) return hipSuccess;
  if (dtype == SPEC_DTYPE_BF16) {
    const int blocks = rows / 16;
    // normalized inputs feed the QKV, gate/up and LM-head projections; the residual ones
    // (output and down projections) read the attention output / SwiGLU product as stored
    const bool norm = a.ss_in != nullptr;
    switch (epi) {
      case EPI_STORE:
        return norm ? gemm_bf16_nt<EPI_STORE, true>(a, blocks, st) : gemm_bf16_nt<EPI_STORE, false>(a, blocks, st);
      case EPI_RESID: return norm ? hipErrorInvalidValue : gemm_bf16_nt<EPI_RESID, false>(a, blocks, st);
      case EPI_QKV:
        return norm ? gemm_bf16_nt<EPI_QKV, true>(a, blocks, st) : gemm_bf16_nt<EPI_QKV, false>(a, blocks, st);
      default:
        return norm ? gemm_bf16_nt<EPI_SWIGLU, true>(a, blocks, st) : gemm_bf16_nt<EPI_SWIGLU, false>(a, blocks, st);
    }
  }
  const int blocks = (rows + 3) / 4;
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, dim3(blocks), dim3(256), 0, st, a); break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_f32_kernel<EPI_RESID>, dim3(blocks), dim3(256), 0, st, a); break;
    case EPI_QKV: hipLaunchKernelGGL(gemm_f32_kernel<EPI_QKV>, dim3(blocks), dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL(gemm_f32_kernel<EPI_SWIGLU>, dim3(blocks), dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st) {
  const int hd = a.cache.hd, G = a.n_q / a.cache.n_kv, R = a.rm.mseq * G;
  const size_t lds = sizeof(float) * ((size_t)R * hd + (size_t)ATTN_CHUNK * (hd + 1) +
                                      (size_t)ATTN_CHUNK * hd + (size_t)R * ATTN_CHUNK + 2 * (size_t)R);
  const int batch = a.rm.M / a.rm.mseq;
  dim3 g1(a.ngrid > 0 ? std::min(a.ngrid, a.nchunk) : a.nchunk, a.cache.n_kv, batch);
  dim3 g2(a.rm.M * a.n_q);
  if (dtype == SPEC_DTYPE_BF16) {
    const int QT = (R + 15) / 16;
    const size_t lds2 = 2 * ((size_t)QT * 16 * (hd + 8) + (size_t)ATTN_CHUNK * (hd + 8) + (size_t)hd * (ATTN_CHUNK + 8));
    if (a.few && hd == 128 && R <= ATTN_FEW_ROWS) {
      hipLaunchKernelGGL(attn_chunk_few_kernel, g1, dim3(256), 0, st, a);
    } else if (QT == 1 && hd == 128) {
      hipLaunchKernelGGL((attn_chunk_mfma_kernel<128, 1>), g1, dim3(256), lds2, st, a);
    } else if (QT <= 2) {
      if (hd == 128) hipLaunchKernelGGL((attn_chunk_mfma_kernel<128, 2>), g1, dim3(256), lds2, st, a);
      else if (hd == 64) hipLaunchKernelGGL((attn_chunk_mfma_kernel<64, 2>), g1, dim3(256), lds2, st, a);
      else hipLaunchKernelGGL((attn_chunk_mfma_kernel<32, 2>), g1, dim3(256), lds2, st, a);
    } else if (hd == 128 && QT == 3) {
      // (the query loads and their registers scale with the instance's tile count)
      hipLaunchKernelGGL((attn_chunk_mfma_kernel<128, 3>), g1, dim3(256), lds2, st, a);
    } else if (hd == 128 && QT == 4) {
      hipLaunchKernelGGL((attn_chunk_mfma_kernel<128, 4>), g1, dim3(256), lds2, st, a);
    } else {
      if (hd == 128) hipLaunchKernelGGL((attn_chunk_mfma_kernel<128, 6>), g1, dim3(256), lds2, st, a);
      else if (hd == 64) hipLaunchKernelGGL((attn_chunk_mfma_kernel<64, 6>), g1, dim3(256), lds2, st, a);
      else hipLaunchKernelGGL((attn_chunk_mfma_kernel<32, 6>), g1, dim3(256), lds2, st, a);
    }
    hipLaunchKernelGGL(attn_combine_kernel<SPEC_DTYPE_BF16>, g2, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(attn_chunk_kernel<SPEC_DTYPE_F32>, g1, dim3(256), lds, st, a);
    hipLaunchKernelGGL(attn_combine_kernel<SPEC_DTYPE_F32>, g2, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

size_t attention_lds_bytes(int R, int hd) {
  return sizeof(float) * ((size_t)R * hd + (size_t)ATTN_CHUNK * (hd + 1) + (size_t)ATTN_CHUNK * hd +
                          (size_t)R * ATTN_CHUNK + 2 * (size_t)R);
}

hipError_t launch_fill(void* p, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(fill_kernel, dim3(blocks), dim3(256), 0, st, (uint32_t*)p, n);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const int32_t* src, int src_ld, int32_t* dst, int n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, src, src_ld, dst, n);
  return hipGetLastError();
}

hipError_t attention_set_lds_limit() {
  const int bytes = 160 * 1024;
  hipError_t e = hipFuncSetAttribute((const void*)attn_chunk_kernel<SPEC_DTYPE_BF16>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)attn_chunk_kernel<SPEC_DTYPE_F32>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t launch_kv_load(int dtype, const void* k, const void* v, CacheView c, int seq, int length,
                          hipStream_t st) {
  if (length == 0) return hipSuccess;
  const int64_t n = (int64_t)c.n_layers * c.n_kv * length * c.hd;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 16384);
  if (dtype == SPEC_DTYPE_BF16)
    hipLaunchKernelGGL(kv_load_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, (const bf16_t*)k,
                       (const bf16_t*)v, c, seq, length);
  else
    hipLaunchKernelGGL(kv_load_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)k,
                       (const float*)v, c, seq, length);
  return hipGetLastError();
}

hipError_t launch_set_len(int32_t* len, int seq, int value, hipStream_t st) {
  hipLaunchKernelGGL(set_len_kernel, dim3(1), dim3(1), 0, st, len, seq, value);
  return hipGetLastError();
}

hipError_t launch_add_len(int32_t* len, int batch, int delta, hipStream_t st) {
  hipLaunchKernelGGL(add_len_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, len, batch, delta);
  return hipGetLastError();
}

}  // namespace spec
