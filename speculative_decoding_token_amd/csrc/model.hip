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
#include "kernels.h"

namespace spec {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

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
// Row m = (seq b, i): token first[b*first_ld] for i == 0, else rest[b*rest_ld + i-1].
template <int DT>
__global__ __launch_bounds__(256) void embed_kernel(const void* E, int d, int vocab,
                                                    const int32_t* first, int first_ld,
                                                    const int32_t* rest, int rest_ld, int mseq,
                                                    float* x) {
  using A = Act<DT>;
  const int m = blockIdx.x, b = m / mseq, i = m % mseq;
  const int tok = (i == 0) ? first[(int64_t)b * first_ld] : rest[(int64_t)b * rest_ld + i - 1];
  const bool ok = tok >= 0 && tok < vocab;
  const typename A::T* row = (const typename A::T*)E + (int64_t)(ok ? tok : 0) * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x)
    x[(int64_t)m * d + c] = ok ? A::load(row, c) : __builtin_nanf("");
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
constexpr int GEMM_NW = 8;
constexpr int GEMM_U = 8;

template <int EPI, int NT>
__global__ __launch_bounds__(GEMM_NW * 64) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int TILES = (EPI == EPI_SWIGLU) ? 2 : 1;
  __shared__ f32x4_t red[GEMM_NW][TILES][NT][64];
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
  const bf16_t* wp[TILES];
  wp[0] = (const bf16_t*)a.w[mat] + (int64_t)(r0 + (lane & 15)) * K + koff;
  if (TILES == 2) wp[TILES - 1] = (const bf16_t*)a.w[1] + (int64_t)(r0 + (lane & 15)) * K + koff;
  const bf16_t* xp[NT];
  bool xv[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int m = nt * 16 + (lane & 15);
    xv[nt] = m < M;
    xp[nt] = (const bf16_t*)a.x + (int64_t)(xv[nt] ? m : 0) * K + koff;
  }
  f32x4_t acc[TILES][NT];
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[t][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int s0 = wave; s0 < nsteps; s0 += GEMM_NW * GEMM_U) {
    uint4 wa[TILES][GEMM_U];
    uint4 xb[NT][GEMM_U];
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u) {
      const int s = s0 + u * GEMM_NW;
      const bool ok = s < nsteps;
#pragma unroll
      for (int t = 0; t < TILES; ++t)
        wa[t][u] = ok ? *(const uint4*)(wp[t] + (int64_t)s * 32) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        xb[nt][u] = (ok && xv[nt]) ? *(const uint4*)(xp[nt] + (int64_t)s * 32) : make_uint4(0, 0, 0, 0);
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
  }
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) red[wave][t][nt][lane] = acc[t][nt];
  __syncthreads();

  // D layout of the 16x16 MFMA: lane l holds column l%16 (token), rows 4*(l/16)+r (weight row)
  for (int e = threadIdx.x; e < NT * 256; e += GEMM_NW * 64) {
    const int nt = e >> 8, l = (e >> 2) & 63, r = e & 3;
    float v[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < GEMM_NW; ++w) s += red[w][t][nt][l][r];
      v[t] = s;
    }
    const int m = nt * 16 + (l & 15);
    const int n = r0 + 4 * (l >> 4) + r;
    if (m < M) gemm_epilogue<SPEC_DTYPE_BF16, EPI>(a, mat, m, n, v[0], v[TILES - 1]);
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
template <int DT>
__global__ __launch_bounds__(256) void attn_chunk_kernel(AttnArgs a) {
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

template <int DT>
__global__ void attn_combine_kernel(AttnArgs a) {
  using A = Act<DT>;
  const int row = blockIdx.x, d = threadIdx.x;
  const int hd = a.cache.hd;
  const int m = row / a.n_q, h = row % a.n_q;
  const int b = m / a.rm.mseq, i = m % a.rm.mseq;
  const int pos = a.rm.len[b] + a.rm.pos_off + i;
  const int nch = pos / ATTN_CHUNK + 1;
  const float* P = a.part + (int64_t)row * a.nchunk * (hd + 2);
  float mx = -__builtin_inff();
  for (int c = 0; c < nch; ++c) mx = fmaxf(mx, P[c * (hd + 2) + hd]);
  float den = 0.0f, o = 0.0f;
  for (int c = 0; c < nch; ++c) {
    const float w = expf(P[c * (hd + 2) + hd] - mx);
    den += P[c * (hd + 2) + hd + 1] * w;
    o += P[c * (hd + 2) + d] * w;
  }
  A::store((typename A::T*)a.out, (int64_t)m * a.n_q * hd + h * hd + d, o / den);
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
                        hipStream_t st) {
  if (dtype == SPEC_DTYPE_BF16)
    hipLaunchKernelGGL(embed_kernel<SPEC_DTYPE_BF16>, dim3(M), dim3(256), 0, st, E, d, vocab, first,
                       first_ld, rest, rest_ld, mseq, x);
  else
    hipLaunchKernelGGL(embed_kernel<SPEC_DTYPE_F32>, dim3(M), dim3(256), 0, st, E, d, vocab, first,
                       first_ld, rest, rest_ld, mseq, x);
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

template <int EPI>
static hipError_t gemm_bf16_nt(const GemmArgs& a, int blocks, hipStream_t st) {
  const int M = a.rm.M;
  if (M <= 16)
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI, 1>), dim3(blocks), dim3(GEMM_NW * 64), 0, st, a);
  else if (M <= 32)
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI, 2>), dim3(blocks), dim3(GEMM_NW * 64), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI, 4>), dim3(blocks), dim3(GEMM_NW * 64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t st) {
  int rows = a.rows[0];
  if (epi == EPI_QKV) rows += a.rows[1] + a.rows[2];
  if (a.rm.M == 0 || rows == 0) return hipSuccess;
  if (dtype == SPEC_DTYPE_BF16) {
    const int blocks = rows / 16;
    switch (epi) {
      case EPI_STORE: return gemm_bf16_nt<EPI_STORE>(a, blocks, st);
      case EPI_RESID: return gemm_bf16_nt<EPI_RESID>(a, blocks, st);
      case EPI_QKV: return gemm_bf16_nt<EPI_QKV>(a, blocks, st);
      default: return gemm_bf16_nt<EPI_SWIGLU>(a, blocks, st);
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
  dim3 g1(a.nchunk, a.cache.n_kv, batch);
  dim3 g2(a.rm.M * a.n_q);
  if (dtype == SPEC_DTYPE_BF16) {
    hipLaunchKernelGGL(attn_chunk_kernel<SPEC_DTYPE_BF16>, g1, dim3(256), lds, st, a);
    hipLaunchKernelGGL(attn_combine_kernel<SPEC_DTYPE_BF16>, g2, dim3(hd), 0, st, a);
  } else {
    hipLaunchKernelGGL(attn_chunk_kernel<SPEC_DTYPE_F32>, g1, dim3(256), lds, st, a);
    hipLaunchKernelGGL(attn_combine_kernel<SPEC_DTYPE_F32>, g2, dim3(hd), 0, st, a);
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
