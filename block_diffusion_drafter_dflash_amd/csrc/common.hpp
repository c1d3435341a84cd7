// Device-side helpers shared by the gfx950 kernels of the draft round.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t u16) {
  return __uint_as_float(u16 << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest, ties to even (the hardware conversion).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two fp32 values -> two bf16 in one 32-bit word (low half first), one instruction.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const bf16x2_t v = __builtin_convertvector((float2_t){a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// float64 -> fp32 rounded to odd: the truncation toward zero with its last bit set
// when inexact. Rounding that result to bf16 (to nearest, ties to even) equals
// rounding the float64 value to bf16 directly, because fp32 keeps more than two
// extra bits.
__device__ __forceinline__ float f32_round_odd(double d) {
  float f = (float)d;
  if ((double)f != d && __builtin_isfinite(f)) {
    uint32_t u = __float_as_uint(f);
    if (fabs((double)f) > fabs(d)) u -= 1u;
    u |= 1u;
    f = __uint_as_float(u);
  }
  return f;
}
__device__ __forceinline__ uint32_t bf16_from_double(double d) { return f32_to_bf16(f32_round_odd(d)); }

// Element traits: E elements per 16-byte fragment, KF = k-elements one 16-byte-per-lane
// fragment covers across the four 16-lane groups of a wave.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int E = 4;
  static constexpr int KF = 16;
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
  __device__ static __forceinline__ float round(float x) { return x; }
  __device__ static __forceinline__ float round_d(double x) { return (float)x; }
  __device__ static __forceinline__ void store_d(float* p, double x) { *p = (float)x; }
};
template <> struct Elem<bf16_t> {
  static constexpr int E = 8;
  static constexpr int KF = 32;
  __device__ static __forceinline__ float load1(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ float round(float x) { return bf16_to_f32(f32_to_bf16(x)); }
  __device__ static __forceinline__ float round_d(double x) { return bf16_to_f32(bf16_from_double(x)); }
  __device__ static __forceinline__ void store_d(bf16_t* p, double x) { *p = (bf16_t)bf16_from_double(x); }
};

// Unpack a 16-byte fragment into floats.
__device__ __forceinline__ void unpack(const uint4& v, float* out, float) {
  out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack(const uint4& v, float* out, bf16_t) {
  out[0] = bf16_to_f32(v.x & 0xffffu); out[1] = bf16_to_f32(v.x >> 16);
  out[2] = bf16_to_f32(v.y & 0xffffu); out[3] = bf16_to_f32(v.y >> 16);
  out[4] = bf16_to_f32(v.z & 0xffffu); out[5] = bf16_to_f32(v.z >> 16);
  out[6] = bf16_to_f32(v.w & 0xffffu); out[7] = bf16_to_f32(v.w >> 16);
}
// Pack floats (already representable, or to be rounded) into a 16-byte fragment.
__device__ __forceinline__ uint4 pack(const float* in, float) {
  return make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]),
                    __float_as_uint(in[3]));
}
__device__ __forceinline__ uint4 pack(const float* in, bf16_t) {
  return make_uint4(f32x2_to_bf16x2(in[0], in[1]), f32x2_to_bf16x2(in[2], in[3]),
                    f32x2_to_bf16x2(in[4], in[5]), f32x2_to_bf16x2(in[6], in[7]));
}

// Pack float64 values into a 16-byte fragment, each rounded once to the element type.
__device__ __forceinline__ uint4 pack_d(const double* in, float) {
  return make_uint4(__float_as_uint((float)in[0]), __float_as_uint((float)in[1]), __float_as_uint((float)in[2]),
                    __float_as_uint((float)in[3]));
}
__device__ __forceinline__ uint4 pack_d(const double* in, bf16_t) {
  return make_uint4(f32x2_to_bf16x2(f32_round_odd(in[0]), f32_round_odd(in[1])),
                    f32x2_to_bf16x2(f32_round_odd(in[2]), f32_round_odd(in[3])),
                    f32x2_to_bf16x2(f32_round_odd(in[4]), f32_round_odd(in[5])),
                    f32x2_to_bf16x2(f32_round_odd(in[6]), f32_round_odd(in[7])));
}

// acc[16x16] += A_frag x B_frag over one fragment's KF k-elements.
// Lane l supplies row (l % 16) of A and column (l % 16) of B; lane group l / 16 supplies
// the same k-slots in both, so any assignment of k indices to slots is valid as long as
// A and B use the same one.
__device__ __forceinline__ void mma_frag(floatx4& acc, const uint4& a, const uint4& b, bf16_t) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_frag(floatx4& acc, const uint4& a, const uint4& b, float) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void stg16(void* p, const uint4& v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// Butterfly sums over lane groups (deterministic order).
__device__ __forceinline__ float xor_sum(float v, int width) {
  for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Rotary cos/sin for position pos and pair index j of a head of size d, computed in
// float64 (angles reach ~1e5 rad at long contexts) and returned as float.
__device__ __forceinline__ void rope_cs(int pos, int j, int d, float theta, float& c, float& s) {
  double inv_freq = pow((double)theta, -2.0 * (double)j / (double)d);
  double ang = (double)pos * inv_freq;
  double sd, cd;
  sincos(ang, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

}  // namespace dfl
