// One launch per projection on the weight-streaming projections of stream_core.h (the
// per-step schedule of bf16 forwards over at most 16 rows).
#include <algorithm>

#include "stream_core.h"

namespace spec {
namespace {

template <int EPI, int NST, int WB>
__global__ __launch_bounds__(sk::SNW * 64) void stream_gemm_kernel(StreamArgs a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  if (a.skip && *a.skip) return;
  sk::Gemm<EPI, NST, false, WB>::run(a, sm, 0);
}

template <int EPI, int NST, int WB = 2>
const void* kptr() {
  return (const void*)stream_gemm_kernel<EPI, NST, WB>;
}

// Resident-slice variants: K = NST * KS for K in {1024, 2048, 3072, 4096, 5120} (bf16); fp8: K in
// {2048, 4096}, and streamed inputs only for the residual epilogue.
int nst_of(int epi, int K, int wbytes) {
  const int ks = (epi == EPI_SWIGLU ? 512 : 1024) * (wbytes == 1 ? 2 : 1);
  if (K % ks) return -1;
  const int n = K / ks;
  if (wbytes == 1) {
    if (K == 2048 || K == 4096) return n;
    return epi == EPI_RESID ? 0 : -1;
  }
  const int k1 = K / 1024;
  if (K % 1024 == 0 && k1 >= 1 && k1 <= 5) return n;
  return 0;
}

template <int EPI>
const void* kernel_for(int nst) {
  constexpr int T = EPI == EPI_SWIGLU ? 2 : 1;
  switch (nst / T) {
    case 1: return kptr<EPI, T * 1>();
    case 2: return kptr<EPI, T * 2>();
    case 3: return kptr<EPI, T * 3>();
    case 4: return kptr<EPI, T * 4>();
    case 5: return kptr<EPI, T * 5>();
    default: return nullptr;
  }
}

// fp8 instances: the stage covers twice the k of a bf16 stage
const void* select_fp8(int epi, int nst) {
  switch (epi) {
    case EPI_STORE: return nst == 1 ? kptr<EPI_STORE, 1, 1>() : (nst == 2 ? kptr<EPI_STORE, 2, 1>() : nullptr);
    case EPI_RESID:
      return nst == 0 ? kptr<EPI_RESID, 0, 1>()
                      : (nst == 1 ? kptr<EPI_RESID, 1, 1>() : (nst == 2 ? kptr<EPI_RESID, 2, 1>() : nullptr));
    case EPI_QKV: return nst == 1 ? kptr<EPI_QKV, 1, 1>() : (nst == 2 ? kptr<EPI_QKV, 2, 1>() : nullptr);
    default: return nst == 2 ? kptr<EPI_SWIGLU, 2, 1>() : (nst == 4 ? kptr<EPI_SWIGLU, 4, 1>() : nullptr);
  }
}

const void* select(int epi, int nst, int wbytes) {
  if (wbytes == 1) return select_fp8(epi, nst);
  if (nst == 0) {
    switch (epi) {
      case EPI_STORE: return kptr<EPI_STORE, 0>();
      case EPI_RESID: return kptr<EPI_RESID, 0>();
      case EPI_QKV: return kptr<EPI_QKV, 0>();
      default: return kptr<EPI_SWIGLU, 0>();
    }
  }
  switch (epi) {
    case EPI_STORE: return kernel_for<EPI_STORE>(nst);
    case EPI_RESID: return kernel_for<EPI_RESID>(nst);
    case EPI_QKV: return kernel_for<EPI_QKV>(nst);
    default: return kernel_for<EPI_SWIGLU>(nst);
  }
}

}  // namespace

bool stream_supported(int M, int K, int epi, bool norm, int wbytes, int units_per_wg) {
  if (M < 1 || M > 32 || (wbytes != 1 && wbytes != 2)) return false;
  const int nst = nst_of(epi, K, wbytes);
  if (nst < 0) return false;
  if (wbytes == 1 && units_per_wg * (epi == EPI_SWIGLU ? 2 : 1) * 16 > sk::SCALE_MAX) return false;
  return !norm || nst > 0;  // normalized inputs need the resident slices
}

size_t stream_lds_bytes() { return (size_t)sk::LDS_BYTES; }

hipError_t stream_init() {
  const int lds = (int)stream_lds_bytes();
  for (int epi : {EPI_STORE, EPI_RESID, EPI_QKV, EPI_SWIGLU}) {
    for (int k1 : {0, 1, 2, 3, 4, 5}) {
      const void* k = select(epi, k1 * (epi == EPI_SWIGLU ? 2 : 1), 2);
      const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
    }
    for (int nst : {0, 1, 2, 4}) {
      const void* k = select(epi, nst, 1);
      if (!k) continue;
      const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_stream_gemm(int epi, const StreamArgs& a, int grid, hipStream_t st) {
  if (a.nunits < 1 || grid < 1) return hipErrorInvalidValue;
  const int g = std::min(grid, a.nunits);
  const int wb = a.wbytes == 1 ? 1 : 2;
  if (!stream_supported(a.M, a.K, epi, a.ss_in != nullptr, wb, (a.nunits + g - 1) / g)) return hipErrorInvalidValue;
  // resident inputs: the residual projections take bf16 rows, the others an RMSNorm input
  if (nst_of(epi, a.K, wb) > 0 && (a.ss_in != nullptr) != (epi != EPI_RESID)) return hipErrorInvalidValue;
  if (wb == 1 && (!a.w0s || (epi == EPI_SWIGLU && !a.w1s) || (epi == EPI_QKV && (!a.w1s || !a.w2s))))
    return hipErrorInvalidValue;
  const void* k = select(epi, nst_of(epi, a.K, wb), wb);
  if (!k) return hipErrorInvalidValue;
  // more than 16 rows: passes of at most 16 (rows 0..15, then the rest), each its own launch
  // over the whole weight stream, every row computed as in a single pass
  for (int r0 = 0; r0 < a.M; r0 += 16) {
    StreamArgs copy = a;
    copy.wbytes = wb;
    copy.M = std::min(16, a.M - r0);
    copy.row0 = a.row0 + r0;
    if (r0 > 0) {
      const int64_t xr = (int64_t)r0 * a.K * (a.ss_in ? 4 : 2);
      copy.x = (const char*)a.x + xr;
      if (a.ss_in) copy.ss_in = a.ss_in + (int64_t)r0 * a.ss_ld;
      if (a.out) copy.out = a.out + (int64_t)r0 * a.ld;
      if (a.ss_out) copy.ss_out = a.ss_out + (int64_t)r0 * a.ss_ld;
      if (a.y_out) copy.y_out = (float*)a.y_out + (int64_t)r0 * a.ld;
      if (a.h) copy.h = (bf16_t*)a.h + (int64_t)r0 * a.rows0;
      if (a.q_stage) copy.q_stage = a.q_stage + (int64_t)r0 * a.rows0;
      if (a.k_stage) copy.k_stage = a.k_stage + (int64_t)r0 * a.rows1;
    }
    void* args[] = {&copy};
    const hipError_t e = hipLaunchKernel(k, dim3(g), dim3(sk::SNW * 64), args, stream_lds_bytes(), st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace spec
