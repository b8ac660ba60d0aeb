// Device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, b);
}

// E4M3 encoding of block-scaled values: codes of the quotients v / s,
// rounded to nearest even by v_cvt_pk_fp8_f32, 8 values to two words.
// Each quotient is v·r corrected once by its residual v − s·(v·r), which one
// FMA gives exactly, with r the correctly rounded 1/s: that is the correctly
// rounded quotient wherever it is a normal number (Markstein's theorem), and
// where it underflows a value with the same E4M3 code (±0, v's sign). So the
// codes are those of the exact division, at a multiply and two FMAs per value
// instead of a division (checked against the division's codes for every fp32
// v with |v| <= 448 s, for scales across the fp32 range; the test
// fp8_quotient_check.c repeats it for six). Scales outside [2^-125, 2^125],
// where r or the residual leaves the normal range, divide outright.
__device__ __forceinline__ bool fp8_fast_scale(float s) { return s >= 0x1p-125f && s <= 0x1p125f; }
__device__ __forceinline__ float fp8_quot(float v, float s, float r) {
  const float y = v * r;
  return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-s, y, v), r, y), v);
}
__device__ __forceinline__ u32x2 fp8_pack8(const float* q) {
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], lo, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], hi, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
  return u32x2{lo, hi};
}
// one scale s for the 8 values (r = 1/s, fast = fp8_fast_scale(s))
__device__ __forceinline__ u32x2 fp8_encode8(const float* v, float s, float r, bool fast) {
  float q[8];
  if (fast) {
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = fp8_quot(v[e], s, r);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = v[e] / s;
  }
  return fp8_pack8(q);
}
// a scale per value (fast: every s[e] passes fp8_fast_scale)
__device__ __forceinline__ u32x2 fp8_encode8(const float* v, const float* s, const float* r, bool fast) {
  float q[8];
  if (fast) {
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = fp8_quot(v[e], s[e], r[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = v[e] / s[e];
  }
  return fp8_pack8(q);
}

// MXFP8 shared exponent of a block of 32 elements with largest magnitude
// amax (>= 0): the smallest x in [-127, 127] with amax * 2^-x <= 448, 0 for
// amax = 0. With amax = 1.m * 2^(E-127): x = E - 134 when the mantissa
// exceeds 0.75 (amax's fraction m/2 above 0.875), else E - 135; an fp32
// subnormal amax gives x below -127, i.e. -127.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  if (b == 0) return 0;
  const int E = int(b >> 23);
  if (E == 0) return -127;
  const int x = E - 134 - ((b & 0x7fffffu) <= 0x600000u ? 1 : 0);
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// E4M3 codes of 8 values scaled by 2^-x (exact), round to nearest even.
__device__ __forceinline__ u32x2 mx_codes8(const float* v, int x) {
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[0], -x), ldexpf(v[1], -x), lo, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[2], -x), ldexpf(v[3], -x), lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4], -x), ldexpf(v[5], -x), hi, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[6], -x), ldexpf(v[7], -x), hi, true);
  return u32x2{lo, hi};
}
// The same with one exponent per value.
__device__ __forceinline__ u32x2 mx_codes8(const float* v, const int* x) {
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[0], -x[0]), ldexpf(v[1], -x[1]), lo, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[2], -x[2]), ldexpf(v[3], -x[3]), lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4], -x[4]), ldexpf(v[5], -x[5]), hi, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[6], -x[6]), ldexpf(v[7], -x[7]), hi, true);
  return u32x2{lo, hi};
}

// Load/store one element of an activation tensor stored as f32 or bf16.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Streaming 16-byte load/store (nontemporal hint). For tensors touched once
// per kernel: the lines do not displace the cache contents of the GEMMs, and
// when the caches hold dirty lines of an earlier kernel these accesses do not
// wait for their write-back (measured on a 100 MB gather-and-sum: 21 us
// instead of 29 us after a 1 GB copy; equal when the caches are clean).
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(q.x, q.y, q.z, q.w);
}
__device__ __forceinline__ void st_stream(void* p, uint4 v) {
  const u32x4 q = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(p));
}

// 16-byte vector of elements: 4 f32 or 8 bf16, unpacked to f32.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const float* p, float* v) {
    float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
  static __device__ __forceinline__ void unpack(uint4 q, float* v) {
    v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
    v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
  }
  static __device__ __forceinline__ uint4 pack(const float* v) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                      __float_as_uint(v[3]));
  }
};
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const bf16_t* p, float* v) {
    uint4 q = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  static __device__ __forceinline__ void unpack(uint4 q, float* v) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Wave-wide reductions (fixed butterfly order: deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

// Bit mask of lanes below this one.
__device__ __forceinline__ uint64_t lanemask_lt() {
  return (uint64_t(1) << lane_id()) - 1;
}

// fp32 exponential used wherever a score must be reproducible bit for bit:
// x = n ln2 + r with n = rint(x log2 e), ln 2 split in a 15-bit leading part
// (so n * hi is exact) and a trailing part, each removed with one fused
// multiply-add; exp(r) by its degree-7 Taylor polynomial (coefficients 1/i!
// rounded to fp32) in Horner form with fused multiply-adds; then scaled by
// 2^n. Inputs above 88 give +inf, below -86 give 0, NaN stays NaN.
__device__ __forceinline__ float exp_spec(float x) {
  if (x != x) return x;
  if (x > 88.0f) return __builtin_inff();
  if (x < -86.0f) return 0.0f;
  const float n = __builtin_rintf(x * 0x1.715476p+0f);
  float r = __builtin_fmaf(-n, 0x1.62e4p-1f, x);
  r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);
  float p = 0x1.a01a02p-13f;
  p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);
  p = __builtin_fmaf(p, r, 0x1.111112p-7f);
  p = __builtin_fmaf(p, r, 0x1.555556p-5f);
  p = __builtin_fmaf(p, r, 0x1.555556p-3f);
  p = __builtin_fmaf(p, r, 0x1p-1f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, static_cast<int>(n));
}

__device__ __forceinline__ float sigmoid_spec(float L) {
  return 1.0f / (1.0f + exp_spec(-L));
}

}  // namespace moe
