// Shared device helpers of the HIP library: number formats, the Philox generator, the
// orderable key of a (value, id) pair, and launch bookkeeping.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spec.h"

#define SPEC_DEVINL __device__ __forceinline__

namespace spec {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;  // one MFMA operand slice
typedef __attribute__((ext_vector_type(4))) float f32x4_t;    // one 16x16 MFMA accumulator slice

// ---- number formats ------------------------------------------------------------------
SPEC_DEVINL float bf16_to_f32(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Round-to-nearest-even float32 -> bfloat16 (gfx950's v_cvt_pk_bf16_f32, one instruction for
// two values); NaN stays NaN.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
SPEC_DEVINL bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
// Two values rounded to bfloat16, lo in the low half of the word.
SPEC_DEVINL uint32_t bf16x2_pack(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---- wavefront reductions without LDS -------------------------------------------------------
// The quad swaps (lane l with l ^ 1, then l ^ 2) and the half-row and row mirrors (DPP) pair the
// lanes within each row of 16; the gfx950 permlane swaps exchange rows 0 <-> 1 and 2 <-> 3 (lane
// l with l ^ 16) and the two halves of the wavefront (l with l ^ 32).  At every step both
// partners already hold one value per group of lanes, so each adds (or takes the larger of) the
// same two values and every lane of the row (of the wavefront) ends with the same result, with
// no LDS round trip.  Callers keep every lane of the wavefront active.
template <int CTRL>
SPEC_DEVINL float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
SPEC_DEVINL float xor16_sum(float x) {  // x[l] + x[l ^ 16]
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}
SPEC_DEVINL float xor32_sum(float x) {  // x[l] + x[l ^ 32]
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}
SPEC_DEVINL float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
SPEC_DEVINL float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
SPEC_DEVINL float row16_sum(float x) {  // over each row of 16 lanes
  x += dpp_f32<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f32<0x141>(x);  // row_half_mirror
  x += dpp_f32<0x140>(x);  // row_mirror
  return x;
}
SPEC_DEVINL float row16_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  x = fmaxf(x, dpp_f32<0x140>(x));
  return x;
}
SPEC_DEVINL float wave_sum(float x) { return xor32_sum(xor16_sum(row16_sum(x))); }
SPEC_DEVINL float wave_max(float x) { return xor32_max(xor16_max(row16_max(x))); }

// Softmax weights of a 64-key attention chunk as A operands of the P V product on the bf16
// MFMA.  Lane l holds query row l % 16 and, in s[kt][r], the score of key 16 kt + 4 (l / 16) + r
// (already scaled, -inf where masked); mx is the row's chunk maximum.  P = exp(s - mx) stays
// float32 up to the product: it is split into hi = bf16(P) and lo = bf16(P - hi) (P - hi is
// exact in float32), so hi + lo carries P to a relative error below 2^-17.  The A operand of
// 32-key step st holds keys 32 st + 4 g + (0..3) in slots 0-3 and 32 st + 16 + 4 g + (0..3) in
// slots 4-7 (g = l / 16); pa[st][0] is the hi part, pa[st][1] the lo part.  Returns the row's
// sum of P over the chunk: the lane's 16 values in order, then the four lane groups.
SPEC_DEVINL float p_operands(const f32x4_t (&s)[4], float mx, bf16x8_t (&pa)[2][2]) {
  uint32_t hi[4][2], lo[4][2];
  float l = 0.0f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    bf16_t h[4], r[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float v = s[kt][rr];
      const float x = (mx == -__builtin_inff() || v == -__builtin_inff()) ? 0.0f : expf(v - mx);
      l += x;
      h[rr] = f32_to_bf16(x);
      r[rr] = f32_to_bf16(x - bf16_to_f32(h[rr]));
    }
    hi[kt][0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    hi[kt][1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
    lo[kt][0] = (uint32_t)r[0] | ((uint32_t)r[1] << 16);
    lo[kt][1] = (uint32_t)r[2] | ((uint32_t)r[3] << 16);
  }
  l = xor32_sum(xor16_sum(l));
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    pa[st][0] = __builtin_bit_cast(bf16x8_t, make_uint4(hi[2 * st][0], hi[2 * st][1], hi[2 * st + 1][0], hi[2 * st + 1][1]));
    pa[st][1] = __builtin_bit_cast(bf16x8_t, make_uint4(lo[2 * st][0], lo[2 * st][1], lo[2 * st + 1][0], lo[2 * st + 1][1]));
  }
  return l;
}

// Activation storage: bf16 models round GEMM inputs and the cache to bfloat16, f32
// models keep float32.
template <int DT> struct Act;
template <> struct Act<SPEC_DTYPE_F32> {
  typedef float T;
  static SPEC_DEVINL float load(const float* p, int64_t i) { return p[i]; }
  static SPEC_DEVINL void store(float* p, int64_t i, float v) { p[i] = v; }
  static SPEC_DEVINL float round(float v) { return v; }
};
template <> struct Act<SPEC_DTYPE_BF16> {
  typedef bf16_t T;
  static SPEC_DEVINL float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static SPEC_DEVINL void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
  static SPEC_DEVINL float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// ---- Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) ----------------------------------
// Ten rounds; each multiplies counter words 0 and 2 by fixed odd constants, swaps in the
// high halves xor-ed with words 1, 3 and the round key, and advances the key by the two
// Weyl increments between rounds.
SPEC_DEVINL uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Uniform in [0, 1 - 2^-24] for counter (slot, round, seq, stream) under key `seed`.
SPEC_DEVINL float philox_uniform(uint64_t seed, uint32_t slot, uint32_t rnd, uint32_t seq,
                                 uint32_t stream) {
  const uint4 o = philox4x32_10(make_uint4(slot, rnd, seq, stream), (uint32_t)seed,
                                (uint32_t)(seed >> 32));
  return (float)(o.x >> 8) * (1.0f / 16777216.0f);
}

enum : uint32_t { STREAM_DRAFT = 0, STREAM_ACCEPT = 1, STREAM_RESIDUAL = 2 };

// ---- ordering of (value, id) ------------------------------------------------------------
// A 64-bit key that is larger for a larger value and, among equal values, for a lower id.
// The value is made +0 when it is -0 so that zeros of both signs tie on id.  0 is never a
// key of a real value (it would be a NaN pattern) and marks an empty slot.
SPEC_DEVINL uint64_t order_key(float z, uint32_t id) {
  z = (z == 0.0f) ? 0.0f : z;
  const uint32_t f = __float_as_uint(z);
  const uint32_t k32 = (f & 0x80000000u) ? ~f : (f | 0x80000000u);
  return ((uint64_t)k32 << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
SPEC_DEVINL float key_value(uint64_t key) {
  const uint32_t k32 = (uint32_t)(key >> 32);
  const uint32_t f = (k32 & 0x80000000u) ? (k32 & 0x7FFFFFFFu) : ~k32;
  return __uint_as_float(f);
}
SPEC_DEVINL uint32_t key_id(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)key; }

constexpr float NEAR_TIE = 1e-6f;

}  // namespace spec
