// The recurrent state of a linear-attention (gated delta rule) layer under speculation.
//
// "Speculative Decoding on Apple Silicon: 119% Faster...", section "Why this needed a patch to
// mlx_lm at all": such a layer cannot drop rejected tokens from a key/value list; it restores
// the state from before the speculative forward and runs the accepted tokens through the
// recurrence again.  Here one launch per verify does both halves: it first folds the tokens
// that the previous verify kept into the committed state and writes that state back, then
// runs the new tokens from it without writing it.  The state is read once and written once per
// cycle and no snapshot is copied: the committed state is the snapshot.
//
// Per head and token (d_k = 128 columns, d_v rows), row i of the state:
//   s_i <- alpha s_i + beta (v_i - alpha (s_i . k)) k,   o_i = s_i . q
// which is S (alpha (I - beta k k^T)) + beta v k^T written row by row.
#include "kernels.h"

namespace spec {
namespace {

constexpr int DK = GDN_DK;
constexpr int RW = 8;        // value rows per wavefront
constexpr int RB = 4 * RW;   // value rows per workgroup (four wavefronts)
constexpr int CL = DK / 8;   // columns per lane: eight lanes share a row

// Sum over the eight lanes of a row group (lanes 8g .. 8g + 7) with DPP moves: swap
// neighbours, swap pairs, then mirror the two quads.  Each step adds a lane's value to its
// partner's and float addition commutes, so all eight lanes end with the same bits.
SPEC_DEVINL float sum8(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
  return x;
}

// Workgroup (row block, head): wavefront w owns rows r0 + 8 w .. + 7; lane l holds columns
// 16 (l % 8) .. + 15 of row l / 8.  Every token's k, q, the block's v rows and the gates are
// staged in LDS first (one round of loads); the token loop then reads only LDS.  A row's dot
// products are 16 products per lane and sum8, an order fixed by the row's data alone, so the
// state after a token is the same whether the token is committed or run speculatively.
__global__ __launch_bounds__(256) void gdn_kernel(GdnArgs a) {
  extern __shared__ __attribute__((aligned(16))) float gsm[];
  const int T = a.n_commit + a.n_fwd;
  const int H = a.n_heads, dv = a.d_v, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = blockIdx.x * RB;
  float* ks = gsm;                  // [T][DK]
  float* qs = ks + T * DK;          // [T][DK]
  float* vs = qs + T * DK;          // [T][RB]
  float* gs = vs + T * RB;          // [T][2] alpha, beta

  for (int e = tid; e < T * DK; e += 256) {
    const int t = e / DK, c = e % DK;
    const int64_t src = ((int64_t)t * H + h) * DK + c;
    ks[e] = a.k[src];
    qs[e] = t >= a.n_commit ? a.q[src] : 0.0f;
  }
  for (int e = tid; e < T * RB; e += 256) {
    const int t = e / RB, r = e % RB;
    vs[e] = a.v[((int64_t)t * H + h) * dv + rb + r];
  }
  for (int t = tid; t < T; t += 256) {
    gs[2 * t] = a.alpha[(int64_t)t * H + h];
    gs[2 * t + 1] = a.beta[(int64_t)t * H + h];
  }
  const int rw = lane >> 3, c0 = (lane & 7) * CL;
  const int row = rb + wave * RW + rw;  // this lane's value row
  float* S = a.state + ((int64_t)h * dv + row) * DK + c0;
  float s[CL];
#pragma unroll
  for (int j = 0; j < CL; j += 4) {
    const float4 x = *(const float4*)(S + j);
    s[j] = x.x;
    s[j + 1] = x.y;
    s[j + 2] = x.z;
    s[j + 3] = x.w;
  }
  __syncthreads();

  auto update = [&](int t) {
    const float* kt = ks + t * DK + c0;
    float kk[CL];
#pragma unroll
    for (int j = 0; j < CL; ++j) kk[j] = kt[j];
    float d = 0.0f;
#pragma unroll
    for (int j = 0; j < CL; ++j) d += s[j] * kk[j];
    d = sum8(d);
    const float al = gs[2 * t], be = gs[2 * t + 1];
    const float u = be * (vs[t * RB + wave * RW + rw] - al * d);
#pragma unroll
    for (int j = 0; j < CL; ++j) s[j] = al * s[j] + u * kk[j];
  };
  for (int t = 0; t < a.n_commit; ++t) update(t);
  if (a.n_commit > 0) {
#pragma unroll
    for (int j = 0; j < CL; j += 4) *(float4*)(S + j) = make_float4(s[j], s[j + 1], s[j + 2], s[j + 3]);
  }
  for (int i = 0; i < a.n_fwd; ++i) {
    const int t = a.n_commit + i;
    update(t);
    const float* qt = qs + t * DK + c0;
    float o = 0.0f;
#pragma unroll
    for (int j = 0; j < CL; ++j) o += s[j] * qt[j];
    o = sum8(o);
    if ((lane & 7) == 0) a.out[((int64_t)i * H + h) * dv + row] = o;
  }
}

}  // namespace

size_t gdn_lds_bytes(int tokens) { return (size_t)tokens * (2 * DK + RB + 2) * sizeof(float); }

hipError_t gdn_init() {
  return hipFuncSetAttribute((const void*)gdn_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)gdn_lds_bytes(GDN_MAX_TOKENS));
}

hipError_t launch_gdn(const GdnArgs& a, hipStream_t st) {
  const int T = a.n_commit + a.n_fwd;
  if (T < 1 || T > GDN_MAX_TOKENS || a.n_heads < 1 || a.d_v < RB || a.d_v % RB) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gdn_kernel, dim3(a.d_v / RB, a.n_heads), dim3(256), gdn_lds_bytes(T), st, a);
  return hipGetLastError();
}

}  // namespace spec
