// Projections of a draft model's one- and two-row forwards on the vector ALUs.
//
// A draft step runs the small model one token at a time ("Speculative Decoding on Apple Silicon:
// 119% Faster...", section "The original result: Qwen3-8B and a 0.6B draft": draft passes are
// sequential, and their cost grows with K), so each projection moves a few MB of weights for one
// or two rows.  A 16-row MFMA tile would be 7/8 or 15/16 padding, which costs nothing by itself,
// but the weight-streaming kernels' LDS ring takes several stage round trips to fill and drain,
// which at 4-13 MB per projection is most of the launch.  Here every weight and input load of a
// workgroup is issued at once, so a projection waits for about one memory round trip:
//
// * one workgroup of 4 wavefronts per unit of 16 weight rows (SwiGLU: 16 gate and 16 up rows);
//   wavefront w holds rows 4w .. 4w+3 of each tile over the whole reduction length K = NK * 512,
//   lane l the 16-byte pieces k = (c * 64 + l) * 8 .. + 7 for c < NK;
// * the input rows (M <= 2) are loaded for the same k; an RMSNorm input arrives as the float32
//   rows x * g, and each wavefront adds the rows' sum-of-squares partials into 1/rms itself (no
//   workgroup barrier before the arithmetic) and rounds (x * g) / rms to bf16, the contract's
//   rounding point;
// * float32 products summed per lane in k order, then across the wavefront by a fixed
//   butterfly of DPP and permlane moves (no LDS); the 16 results per row and tile meet in LDS
//   for the epilogues of the streamed projections (residual add with sum-of-squares partials
//   and the next norm's x * g, SwiGLU, q / k staging and the value rows into the cache).
//
// A row's result depends only on that row, so a two-row forward computes each row exactly as a
// one-row forward does.
#include "stream_core.h"

namespace spec {
namespace {

constexpr int GV_RW = 4;       // rows per wavefront and tile
constexpr int GV_WAVES = 4;
constexpr int GV_MAX_M = 2;

template <int EPI, int NK, bool NORM>
__global__ __launch_bounds__(GV_WAVES * 64) void gemv_kernel(StreamArgs a) {
  constexpr int T = EPI == EPI_SWIGLU ? 2 : 1;
  constexpr int K = NK * 512;
  __shared__ float s_out[T][16][GV_MAX_M];
  __shared__ float s_sq[GV_MAX_M][16];
  const int u = blockIdx.x, tx = threadIdx.x, lane = tx & 63, wave = tx >> 6;
  const int M = a.M;

  // The epilogue's thread e < 16 M takes column ec = e % 16 of the unit for input row em = e / 16.
  // Its operands from memory (the residual and the next norm's gain, the cache position of a
  // value row) are loaded here, ahead of the weights, so that the epilogue waits for no second
  // round trip after the products.
  const int e = tx, em = e >> 4, ec = e & 15;
  const bool live = e < 16 * M;
  int mat = 0, r0 = 0;
  (void)sk::unit_rows<EPI, 2>(a, u, 0, &mat, &r0);
  const int n = r0 + ec;
  // Every thread loads (the others from row 0, unused), and the values are kept as loaded, so
  // that no branch or arithmetic puts a wait for them ahead of the weight loads.
  float res = 0.0f;
  bf16_t gain_b = 0;
  int vlen = 0;
  if (EPI == EPI_RESID) {
    // without a next norm the gain load reads the residual's own first bytes, unused
    const float* res_p = a.out + (int64_t)(live ? em : 0) * a.ld + n;
    res = *res_p;
    gain_b = *(a.y_out ? (const bf16_t*)a.y_gain + n : (const bf16_t*)res_p);
  }
  // (sequence em / mseq of row em < 2 is em >= mseq: no integer division ahead of the weights)
  if (EPI == EPI_QKV && mat == 2) vlen = a.rm.len[live && em >= a.rm.mseq ? 1 : 0];

  // weights: rows r0 + 4 wave + i of each tile, pieces c of 16 bytes
  uint4 w[T][GV_RW][NK];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    int mat, r0;
    const char* base = sk::unit_rows<EPI, 2>(a, u, t, &mat, &r0);
#pragma unroll
    for (int i = 0; i < GV_RW; ++i) {
      const char* row = base + (int64_t)(GV_RW * wave + i) * K * 2;
#pragma unroll
      for (int c = 0; c < NK; ++c)
        w[t][i][c] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const __attribute__((address_space(1))) sk::u32x4_t*)(row + (int64_t)(c * 64 + lane) * 16)));
    }
  }
  // inputs: bf16 rows, or float32 rows x * g of an RMSNorm input with its partials
  constexpr bool norm = NORM;
  uint4 xb[GV_MAX_M][NK];
  float xf[NORM ? GV_MAX_M : 1][NORM ? NK : 1][8];
  float ps[NORM ? GV_MAX_M : 1][2];
#pragma unroll
  for (int m = 0; m < GV_MAX_M; ++m) {
    if (m >= M) break;
    if (norm) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int p = lane + 64 * q;
        ps[NORM ? m : 0][q] = p < a.np_in ? a.ss_in[(int64_t)m * a.ss_ld + p] : 0.0f;
      }
#pragma unroll
      for (int c = 0; c < NK; ++c) {
        const float* src = (const float*)a.x + (int64_t)m * K + (c * 64 + lane) * 8;
        const float4 lo = *(const float4*)src, hi = *(const float4*)(src + 4);
        float* d = xf[NORM ? m : 0][NORM ? c : 0];
        d[0] = lo.x; d[1] = lo.y; d[2] = lo.z; d[3] = lo.w;
        d[4] = hi.x; d[5] = hi.y; d[6] = hi.z; d[7] = hi.w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < NK; ++c)
        xb[m][c] = *(const uint4*)((const bf16_t*)a.x + (int64_t)m * K + (c * 64 + lane) * 8);
    }
  }
  // a skipped draft launch leaves here; the check comes after the loads are issued so that
  // the argument it reads is fetched with the others
  if (a.skip && *a.skip) return;
  if (norm) {
    // 1/rms of each input row: lane j adds partials j, j + 64 in order, then the wavefront sum
#pragma unroll
    for (int m = 0; m < GV_MAX_M; ++m) {
      if (m >= M) break;
      const float sum = wave_sum(ps[NORM ? m : 0][0] + ps[NORM ? m : 0][1]);
      const float rinv = 1.0f / sqrtf(sum / (float)K + a.eps);
#pragma unroll
      for (int c = 0; c < NK; ++c) {
        const float* f = xf[NORM ? m : 0][NORM ? c : 0];
        xb[m][c] = make_uint4(bf16x2_pack(f[0] * rinv, f[1] * rinv), bf16x2_pack(f[2] * rinv, f[3] * rinv),
                              bf16x2_pack(f[4] * rinv, f[5] * rinv), bf16x2_pack(f[6] * rinv, f[7] * rinv));
      }
    }
  }
  // products: per lane in k order, then across the wavefront
#pragma unroll
  for (int m = 0; m < GV_MAX_M; ++m) {
    if (m >= M) break;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int i = 0; i < GV_RW; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < NK; ++c) {
          const uint32_t wv[4] = {w[t][i][c].x, w[t][i][c].y, w[t][i][c].z, w[t][i][c].w};
          const uint32_t xv[4] = {xb[m][c].x, xb[m][c].y, xb[m][c].z, xb[m][c].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc = fmaf(__uint_as_float(wv[e] << 16), __uint_as_float(xv[e] << 16), acc);
            acc = fmaf(__uint_as_float(wv[e] & 0xFFFF0000u), __uint_as_float(xv[e] & 0xFFFF0000u), acc);
          }
        }
        acc = wave_sum(acc);
        if (lane == 0) s_out[t][GV_RW * wave + i][m] = acc;
      }
  }
  __syncthreads();
  // epilogue
  const int m = em, c = ec;
  if (EPI == EPI_RESID) {
    float xn = 0.0f;
    if (live) {
      xn = res + s_out[0][c][m];
      a.out[(int64_t)m * a.ld + n] = xn;
      if (a.y_out) ((float*)a.y_out)[(int64_t)m * a.ld + n] = xn * bf16_to_f32(gain_b);
      s_sq[m][c] = xn * xn;
    }
    if (a.ss_out) {
      __syncthreads();
      if (live && c == 0) {
        float sq = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) sq += s_sq[m][j];
        a.ss_out[(int64_t)m * a.ss_ld + u] = sq;
      }
    }
  } else if (live) {
    const float v = s_out[0][c][m];
    if (EPI == EPI_STORE) {
      a.out[(int64_t)m * a.ld + n] = v;
    } else if (EPI == EPI_SWIGLU) {
      ((bf16_t*)a.h)[(int64_t)m * a.rows0 + n] = f32_to_bf16(sk::silu_s(v) * s_out[T - 1][c][m]);
    } else {  // EPI_QKV
      if (mat == 0) {
        a.q_stage[(int64_t)m * a.rows0 + n] = v;
      } else if (mat == 1) {
        a.k_stage[(int64_t)m * a.rows1 + n] = v;
      } else {
        const CacheView& cv = a.cache;
        const int b = m / a.rm.mseq;
        const int pos = vlen + a.rm.pos_off + m % a.rm.mseq;
        const int kvh = n / cv.hd, dd = n % cv.hd;
        const int64_t idx = ((((int64_t)b * cv.n_layers + a.layer) * cv.n_kv + kvh) * cv.cap + pos) * cv.hd + dd;
        ((bf16_t*)cv.v)[idx] = f32_to_bf16(v);
      }
    }
  }
}

// Instances: RMSNorm inputs (QKV, gate/up, vocabulary) over d in {1024, 2048, 4096} (gate/up up
// to 2048), plain inputs (the residual projections) over K in {1024, 2048, 3072, 3584, 4096}.
template <int EPI, bool NORM>
const void* gemv_ptr(int nk) {
  if constexpr (NORM) {
    switch (nk) {
      case 2: return (const void*)gemv_kernel<EPI, 2, NORM>;
      case 4: return (const void*)gemv_kernel<EPI, 4, NORM>;
      case 8: return EPI == EPI_SWIGLU ? nullptr : (const void*)gemv_kernel<EPI, EPI == EPI_SWIGLU ? 4 : 8, NORM>;
      default: return nullptr;
    }
  }
  else switch (nk) {
    case 2: return (const void*)gemv_kernel<EPI, 2, NORM>;
    case 4: return (const void*)gemv_kernel<EPI, 4, NORM>;
    case 6: return (const void*)gemv_kernel<EPI, 6, NORM>;
    case 7: return (const void*)gemv_kernel<EPI, 7, NORM>;
    case 8: return (const void*)gemv_kernel<EPI, 8, NORM>;
    default: return nullptr;
  }
}

const void* gemv_select(int epi, int K, bool norm) {
  if (K % 512) return nullptr;
  const int nk = K / 512;
  switch (epi) {
    case EPI_STORE: return norm ? gemv_ptr<EPI_STORE, true>(nk) : nullptr;
    case EPI_RESID: return norm ? nullptr : gemv_ptr<EPI_RESID, false>(nk);
    case EPI_QKV: return norm ? gemv_ptr<EPI_QKV, true>(nk) : nullptr;
    case EPI_SWIGLU: return norm ? gemv_ptr<EPI_SWIGLU, true>(nk) : nullptr;
    default: return nullptr;
  }
}

}  // namespace

bool gemv_supported(int M, int K, int epi, bool norm, int wbytes) {
  return M >= 1 && M <= GV_MAX_M && wbytes == 2 && gemv_select(epi, K, norm) != nullptr;
}

hipError_t launch_gemv(int epi, const StreamArgs& a, hipStream_t st) {
  const bool norm = a.ss_in != nullptr;
  if (!gemv_supported(a.M, a.K, epi, norm, a.wbytes == 1 ? 1 : 2) || a.nunits < 1) return hipErrorInvalidValue;
  if (norm && a.np_in > 128) return hipErrorInvalidValue;
  const void* k = gemv_select(epi, a.K, norm);
  StreamArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(k, dim3(a.nunits), dim3(GV_WAVES * 64), args, 0, st);
}

}  // namespace spec
