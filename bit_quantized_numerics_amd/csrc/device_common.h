// device_common.h -- gfx950 device helpers shared by the NVFP4 kernels.
//
// Citations: [Review] = web page "NVFP4 4-bit Pretraining, Made Practical: 12B
// up to 10T Tokens, Effectively On Par with FP8" (review of arXiv 2509.25149),
// by numbered section; [Captions] = that paper's figure-caption list.
//
// Every fp32 step that decides a code is one IEEE operation rounded to nearest
// even, in the order the C ABI header states (the library is built with
// -ffp-contract=off, IEEE denormals and correctly rounded fp32 division), so
// codes and scales are reproducible bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Status word values (mirror nvfp4_status).
constexpr uint32_t kStatusNonfinite = 7u;
// Bit pattern of +inf: |x| bit patterns at or above it are Inf or NaN.
constexpr uint32_t kInfBits = 0x7F800000u;

// ---------------------------------------------------------------- loads

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight consecutive elements starting at p (16-byte aligned for bf16, 32 for fp32).
__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// ---------------------------------------------------------------- cross-lane

// Value of the neighbouring lane (lane ^ 1) via DPP quad_perm [1,0,3,2].
__device__ __forceinline__ float lane_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

// ---------------------------------------------------------------- scales

// Tensor scales from the amax bit pattern [Review s1 Step 1]:
// s_enc = 2688/amax (saturated at FLT_MAX; 1 for amax 0), s6 = s_enc/6, g = 1/s_enc.
struct TensorScales {
  float s_enc, s6, g;
};
__device__ __forceinline__ TensorScales tensor_scales(uint32_t amax_bits) {
  TensorScales ts;
  const float amax = __uint_as_float(amax_bits);
  if (amax == 0.0f) {
    ts.s_enc = 1.0f;
    ts.g = 1.0f;
    ts.s6 = 1.0f / 6.0f;
    return ts;
  }
  float s = 2688.0f / amax;
  if (__builtin_isinf(s)) s = 3.402823466e38f;
  ts.s_enc = s;
  ts.g = 1.0f / s;
  ts.s6 = s / 6.0f;
  return ts;
}

// E4M3FN encode of a non-negative finite fp32, nearest-even, saturating at
// 448 [Review s1 Step 2].  Returns the code; *val receives its value.
__device__ __forceinline__ uint32_t e4m3_encode(float t, float* val) {
  if (!(t >= 0x1p-6f)) {              // subnormal range, multiples of 2^-9
    const float q = __builtin_rintf(t * 512.0f);  // 0..8, ties to even
    *val = q * 0x1p-9f;
    return (uint32_t)q;               // 8 is the code of 2^-6
  }
  if (t >= 448.0f) {
    *val = 448.0f;
    return 0x7Eu;
  }
  uint32_t b = __float_as_uint(t);
  b += 0x7FFFFu + ((b >> 20) & 1u);   // round the mantissa to 3 bits, ties even
  b &= 0xFFF00000u;
  *val = __uint_as_float(b);
  return (b >> 20) - 960u;            // rebias exponent 127 -> 7
}

// Element multiplier r_b = s_enc / d_b (0 for an all-zero block; saturated).
__device__ __forceinline__ float elem_multiplier(float s_enc, float d) {
  if (d == 0.0f) return 0.0f;
  float r = s_enc / d;
  if (__builtin_isinf(r)) r = 3.402823466e38f;
  return r;
}

// Block scale and multiplier from a block amax.
__device__ __forceinline__ float block_scale(float amax_b, const TensorScales& ts, uint32_t* code) {
  float d;
  *code = e4m3_encode(amax_b * ts.s6, &d);
  return elem_multiplier(ts.s_enc, d);
}

// ---------------------------------------------------------------- E2M1 codes

// Two fp32 values -> two E2M1 codes (nearest-even, saturating, sign of zero
// kept) written into byte SEL of `old`; low nibble = a.  gfx950's convert
// with unit scale performs exactly this rounding.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_rn(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Eight values -> eight nearest-even codes in one dword (value i in nibble i).
// The four converts write all four bytes, so the register the chain starts
// from (v[0]'s, already live) needs no clearing.
__device__ __forceinline__ uint32_t fp4x8_rn(const float* v) {
  uint32_t w = __float_as_uint(v[0]);
  w = fp4x2_rn<0>(w, v[0], v[1]);
  w = fp4x2_rn<1>(w, v[2], v[3]);
  w = fp4x2_rn<2>(w, v[4], v[5]);
  w = fp4x2_rn<3>(w, v[6], v[7]);
  return w;
}

// Stochastic rounding to E2M1 [Review s10 SR formula; s7 SR example]: with
// lo <= |v| < hi the neighbouring grid values and T = floor((|v| - lo) /
// (hi - lo) * 2^22) (the fraction in 22-bit fixed point), round up iff
// 64 * r16 < T; |v| >= 6 gives 6.  gfx950's stochastic FP4 convert of a pair
// (unit scale) rounds element 0 up iff (rnd >> 10) + T >= 2^22 and element 1
// up iff ((rnd << 1) >> 10) + T >= 2^22 (both established by on-GPU sweeps of
// its rounding), so a random operand whose 22-bit field is 2^22 - 1 - 64 r16
// -- ~(r16 << 16) for element 0, ~(r16 << 15) for element 1 -- reproduces the
// rule exactly.  The two fields overlap, so each element of a pair gets its
// own call: the first keeps element 0's code (bits 0..3 of the result), the
// second element 1's (bits 4..7).
__device__ __forceinline__ uint32_t fp4x2_sr(float a, float b, uint32_t ra, uint32_t rb) {
  typedef float float2_t __attribute__((ext_vector_type(2)));
  const float2_t pair = {a, b};
  const uint32_t lo = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, pair, ~(ra << 16), 1.0f, 0);
  const uint32_t hi = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, pair, ~(rb << 15), 1.0f, 0);
  return (lo & 0x0Fu) | (hi & 0xF0u);
}

// ---------------------------------------------------------------- Philox

// Philox4x32-10 (Salmon, Moraes, Dror & Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies with Weyl-sequence key bumps.
struct U4 {
  uint32_t x, y, z, w;
};
__device__ __forceinline__ U4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                            uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // three-input xor (truth table 0x96) in one instruction
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return U4{c0, c1, c2, c3};
}

// Philox4x32-10 with output words 0 and 2 complemented: the last round's
// three-input xor for those words becomes an xnor at no cost (truth table
// 0x69), for callers that want ~word anyway.
__device__ __forceinline__ U4 philox4x32_10_n02(uint32_t c0, uint32_t c1, uint32_t c2,
                                                uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t n0, n2;
    if (r < 9) {
      n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
      n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    } else {
      n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x69);
      n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x69);
    }
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return U4{c0, c1, c2, c3};
}

// The eight 16-bit draws of elements e .. e+7 (e % 8 == 0) of one operand.
__device__ __forceinline__ U4 sr_draw8(uint64_t seed, uint32_t stream, uint64_t e) {
  const uint64_t j = e >> 3;
  return philox4x32_10((uint32_t)j, (uint32_t)(j >> 32), stream, 0u, (uint32_t)seed,
                       (uint32_t)(seed >> 32));
}

// Eight values -> eight SR codes (value i in nibble i) using the eight 16-bit
// draws in r (draw i = half i of the 128-bit output, low half first).
__device__ __forceinline__ uint32_t fp4x8_sr(const float* v, const U4& r) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  uint32_t out = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    out |= fp4x2_sr(v[2 * k], v[2 * k + 1], w[k] & 0xFFFFu, w[k] >> 16) << (8 * k);
  return out;
}

// ---------------------------------------------------------------- block scales (fast path)

// E4M3 code of a block's t = amax_b * s_enc/6 (non-negative, finite): gfx950's
// fp8 convert rounds to nearest-even over the E4M3FN grid, subnormals
// included, but turns values past the largest finite one into NaN, so t is
// first clamped at 448; the pair (t, 0) packs code | 0 << 8 into the low word
// (an on-GPU sweep over 281k values of t, every midpoint of the grid and its
// fp32 neighbours, matched the rounding rule of e4m3_encode exactly).
__device__ __forceinline__ uint32_t e4m3_code(float t) {
  const float c = __builtin_fminf(t, 448.0f);
  // the upper word is left as it was in the destination (unused, masked off)
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, (int)__float_as_uint(c), false) & 0xFFu;
}

// Value of E4M3FN code c (0..126): subnormal m * 2^-9, normal (1 + m/8) 2^(e-7).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// ---------------------------------------------------------------- packed bf16 elements

// Element j (0..7) of a row of 8 bf16 held in 4 dwords, as fp32.
__device__ __forceinline__ float bf16_elem(const uint32_t* w, int j) {
  return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
}
// The same with its sign bit flipped when sm == 0x80000000 (sm is 0 or
// that): (w << 16) + sm for the low half, (w & 0xFFFF0000) ^ sm for the high.
__device__ __forceinline__ float bf16_elem_signed(const uint32_t* w, int j, uint32_t sm) {
  const uint32_t x = w[j >> 1];
  return (j & 1) ? __uint_as_float(__builtin_amdgcn_bitop3_b32(x, 0xFFFF0000u, sm, 0x6A))
                 : __uint_as_float((x << 16) + sm);
}

// ---------------------------------------------------------------- stochastic E2M1 (pairs)

typedef float float2_t __attribute__((ext_vector_type(2)));

// One stochastic FP4 convert of the pair p into byte SEL of `old`, the other
// bytes kept (the instruction writes only the selected byte; the builtin does
// not model that, so it is written out with the destination tied).  The
// trailing s_nop is the one wait state a VALU read of the result needs.
// SEL < 0: byte 0 of a fresh register (the other bytes are left undefined;
// the caller fills them with SEL 1..3).
template <int SEL>
__device__ __forceinline__ uint32_t cvt_sr_byte(uint32_t old, float2_t p, uint32_t rnd) {
  if (SEL < 0)
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0\n\ts_nop 0" : "=v"(old) : "v"(p), "v"(rnd));
  else if (SEL == 0)
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0\n\ts_nop 0" : "+v"(old) : "v"(p), "v"(rnd));
  else if (SEL == 1)
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,0]\n\ts_nop 0"
                 : "+v"(old) : "v"(p), "v"(rnd));
  else if (SEL == 2)
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,0,1]\n\ts_nop 0"
                 : "+v"(old) : "v"(p), "v"(rnd));
  else
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,1]\n\ts_nop 0"
                 : "+v"(old) : "v"(p), "v"(rnd));
  return old;
}

// The eight draws of elements e .. e+7 as sr_draw8, with words 0 and 2
// complemented (see philox4x32_10_n02).
__device__ __forceinline__ U4 sr_draw8_n02(uint64_t seed, uint32_t stream, uint64_t e) {
  const uint64_t j = e >> 3;
  return philox4x32_10_n02((uint32_t)j, (uint32_t)(j >> 32), stream, 0u, (uint32_t)seed,
                           (uint32_t)(seed >> 32));
}

// Eight values -> eight SR codes (value i in nibble i) from the four words of
// one Philox output as sr_draw8_n02 returns it (value 2k takes the low half of
// word k, value 2k+1 the high half), by the rule of fp4x2_sr.  Each pair is
// converted twice with the same operands: once with the even value's draw
// placed for slot 0 (its code lands in the low nibble of byte k of E) and once
// with the odd value's draw placed for slot 1 (high nibble of byte k of O);
// nw = ~word gives both fields: slot 0 reads bits 31..10 = ~lo16 then ones,
// slot 1 bits 30..9 = ~hi16 then ones.
__device__ __forceinline__ uint32_t fp4x8_sr2(const float* v, const U4& r) {
  const uint32_t nws[4] = {r.x, ~r.y, r.z, ~r.w};  // words 0 and 2 arrive complemented
  uint32_t E, O;
#define NVFP4_SR_PAIR(K, SEL)                                         \
  {                                                                   \
    const float2_t p = {v[2 * K], v[2 * K + 1]};                      \
    const uint32_t nw = nws[K];                                       \
    E = cvt_sr_byte<SEL>(E, p, (nw << 16) | 0xFFFFu);                 \
    O = cvt_sr_byte<SEL>(O, p, (nw >> 1) | 0x7E00u);                  \
  }
  NVFP4_SR_PAIR(0, -1) NVFP4_SR_PAIR(1, 1) NVFP4_SR_PAIR(2, 2) NVFP4_SR_PAIR(3, 3)
#undef NVFP4_SR_PAIR
  return (E & 0x0F0F0F0Fu) | (O & 0xF0F0F0F0u);
}

// ---------------------------------------------------------------- RHT16

// In-place 16-point transform y = 1/4 H16 diag(s) x on u[0..15] with stride
// S [Review s3]: signs, butterflies h = 1, 2, 4, 8 as (a+b, a-b), x 1/4.
template <int S>
__device__ __forceinline__ void rht16_inplace(float* u, uint32_t signs) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if ((signs >> i) & 1u) u[i * S] = -u[i * S];
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      const float a = u[i * S], b = u[(i + h) * S];
      u[i * S] = a + b;
      u[(i + h) * S] = a - b;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i * S] = u[i * S] * 0.25f;
}

// In-place 4-point transforms y = 1/2 H4 diag(s) x on the four chunks
// u[0..3], u[4..7], u[8..11], u[12..15] (stride S) with the same four signs
// (bits 0-3) [Review s3; Captions Fig. 12]: signs, butterflies h = 1, 2 as
// (a+b, a-b), x 1/2.
template <int S>
__device__ __forceinline__ void rht4_inplace(float* u, uint32_t signs) {
#pragma unroll
  for (int c = 0; c < 16; c += 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if ((signs >> i) & 1u) u[(c + i) * S] = -u[(c + i) * S];
#pragma unroll
    for (int h = 1; h < 4; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i & h) continue;
        const float a = u[(c + i) * S], b = u[(c + i + h) * S];
        u[(c + i) * S] = a + b;
        u[(c + i + h) * S] = a - b;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) u[(c + i) * S] = u[(c + i) * S] * 0.5f;
  }
}

}  // namespace nvfp4
