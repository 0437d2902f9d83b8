// Device-side building blocks shared by the attention kernels (gfx950).
//
// MFMA operand layouts used throughout (wave64, verified by the parity tests):
//   32x32x16 (bf16/f16): lane l holds A[l%32][k in half l/32] and
//     B[k in half l/32][l%32] (8 values each); accumulator register i of
//     lane l holds C[8*(i/4) + 4*(l/32) + i%4][l%32].
//   16x16x32 (bf16/f16): lane l holds A[l%16][k in quarter l/16] and
//     B[k in quarter l/16][l%16]; accumulator register i holds
//     C[4*(l/16) + i][l%16].
//   32x32x64 f8f6f4: as 32x32x16 with 32 one-byte values per lane.
// Only the M/N placement and the accumulator layout matter to the kernels:
// A and B share the lane-to-k assignment, so any permutation of k within a
// lane group leaves the contraction unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn.h"

namespace attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Raw buffer resources (CDNA buffer descriptors): word 3 selects 32-bit
// untyped data with no swizzle, so the range check is a plain byte-offset
// test and an out-of-range load returns zero without a memory access.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kBufferNontemporal = 2;  // cache-policy bit: streaming (nt)

// ---------------------------------------------------------------------------
// Element types (16-bit storage types are handled as raw bit patterns)
// ---------------------------------------------------------------------------
struct Bf16Tag {
  static constexpr int kBytes = 2;
  __device__ static inline float to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
  // round-to-nearest-even via the hardware convert (v_cvt_pk_bf16_f32)
  __device__ static inline uint32_t pack2(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) __bf16 v2;
    v2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  // acc + lo + hi of a packed pair (v_dot2 with (1, 1))
  __device__ static inline float sum2(uint32_t packed, float acc) {
    typedef __attribute__((ext_vector_type(2))) __bf16 v2;
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2, packed), __builtin_bit_cast(v2, 0x3f803f80u), acc, false);
  }
  __device__ static inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

struct F16Tag {
  static constexpr int kBytes = 2;
  __device__ static inline float to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {  // RNE (v_cvt_pk_f16_f32)
    typedef __attribute__((ext_vector_type(2))) _Float16 v2;
    v2 r;
    r[0] = (_Float16)lo;
    r[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  __device__ static inline float sum2(uint32_t packed, float acc) {
    typedef __attribute__((ext_vector_type(2))) _Float16 v2;
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(v2, packed), __builtin_bit_cast(v2, 0x3c003c00u), acc, false);
  }
  __device__ static inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

// e5m2 -> f16 is exact: an E5M2 byte is the high byte of the f16 with the
// same value (same exponent width and bias, two mantissa bits).
__device__ inline uint32_t e5m2x2_to_f16x2(uint32_t two_bytes) {
  return ((two_bytes & 0xffu) << 8) | ((two_bytes & 0xff00u) << 16);
}

// QK^T on bf8 x bf8 MFMA (A and B both OCP E5M2, unit block scales 2^0).
__device__ inline f32x16 mfma32_bf8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 1, 1, 0, 127, 0, 127);
}
// A in bf8 (e5m2), B in fp8 (e4m3), unit scales
__device__ inline f32x16 mfma32_bf8_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 1, 0, 0, 127, 0, 127);
}

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float wave_max_xor(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask)); }

// 16-byte global load / store of raw bits
__device__ inline u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline u32x2 ldg8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// Store n consecutive fp32 values (n = 4) converted to the output dtype.
__device__ inline void store4(void* base, size_t idx, int out_dtype, float a, float b, float c,
                              float d) {
  if (out_dtype == ATTN_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + idx) = f32x4{a, b, c, d};
  } else if (out_dtype == ATTN_BF16) {
    u32x2 w = {Bf16Tag::pack2(a, b), Bf16Tag::pack2(c, d)};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + idx) = w;
  } else {
    u32x2 w = {F16Tag::pack2(a, b), F16Tag::pack2(c, d)};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + idx) = w;
  }
}

__device__ inline void store1(void* base, size_t idx, int out_dtype, float a) {
  if (out_dtype == ATTN_F32) {
    reinterpret_cast<float*>(base)[idx] = a;
  } else if (out_dtype == ATTN_BF16) {
    reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)Bf16Tag::pack2(a, 0.f);
  } else {
    reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)F16Tag::pack2(a, 0.f);
  }
}

}  // namespace attn

// Host-side helpers shared by the entry points.
namespace attn_host {
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline attn_status launch_status() {
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
// RoPE frequencies theta^(-2i/D) in revolutions per position, f = w / (2 pi),
// split (in double) as f_hi + f_mid + f_lo with f_hi and f_mid carrying 8
// significant bits each: pos * f_hi and pos * f_mid are then exact in fp32
// for pos < 2^16, and pos * f_lo stays below 2^-6 revolutions, so the device
// reduces an angle modulo one revolution as
//   frac(frac(pos f_hi) + frac(pos f_mid) + pos f_lo)
// with an error of a few fp32 ulps of one revolution.  fmid may be null: the
// two-way split f_hi + (f_mid + f_lo) is then returned in fhi / flo.
inline void rope_freq_split(float theta, int D, float* inv_freq, float* fhi, float* flo, float* fmid = nullptr) {
  auto top8 = [](double f) {  // f rounded down to 8 significant bits
    if (f == 0.0) return 0.0;
    int ex = 0;
    const double mant = frexp(f, &ex);  // f = mant * 2^ex, mant in [0.5, 1)
    return ldexp(floor(ldexp(mant, 8)), ex - 8);
  };
  for (int i = 0; i < D / 2; ++i) {
    const double w = pow((double)theta, -2.0 * i / D);
    const double f = w / (2.0 * 3.14159265358979323846);
    const double hi = top8(f);
    if (inv_freq) inv_freq[i] = (float)w;
    fhi[i] = (float)hi;
    if (fmid) {
      const double mid = top8(f - hi);
      fmid[i] = (float)mid;
      flo[i] = (float)(f - hi - mid);
    } else {
      flo[i] = (float)(f - hi);
    }
  }
}
}  // namespace attn_host
