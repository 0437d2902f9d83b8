// Rotation of rotate-half RoPE pairs held as 16-byte chunks, shared by the
// rotation and append kernels and by the chunk-mode prefill kernel (which
// appends the chunk's keys itself and must write bit for bit what the append
// kernel writes).
#pragma once

#include "common.hpp"

namespace attn {

struct F32Elem {
  static constexpr int kBytes = 4;
};

// Rotate the rotate-half pairs held by one 16-byte chunk of the first half
// (lo, elements EPC c .. EPC c + EPC - 1) and its partner chunk D/2 elements
// later (hi) to position pos; fhi/fmid/flo: the three-part split of each
// frequency in revolutions per position.
template <class Tag>
__device__ inline void rotate_chunk_pair(u32x4& lo, u32x4& hi, float pos, int c, const float* fhi,
                                         const float* fmid, const float* flo) {
  constexpr int EB = Tag::kBytes;
  constexpr int EPC = 16 / EB;
  float a[EPC], b[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    if constexpr (EB == 4) {
      a[e] = __uint_as_float(lo[e]);
      b[e] = __uint_as_float(hi[e]);
    } else {
      a[e] = Tag::to_f32((e & 1) ? (lo[e >> 1] >> 16) : (lo[e >> 1] & 0xffff));
      b[e] = Tag::to_f32((e & 1) ? (hi[e >> 1] >> 16) : (hi[e >> 1] & 0xffff));
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    const int i = c * EPC + e;
    // angle in revolutions, reduced to [0, 1) (v_sin / v_cos take revolutions)
    const float rev = __builtin_amdgcn_fractf(__builtin_amdgcn_fractf(pos * fhi[i]) +
                                              __builtin_amdgcn_fractf(pos * fmid[i]) + pos * flo[i]);
    const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
    const float ra = a[e] * cs - b[e] * sn, rb = b[e] * cs + a[e] * sn;
    a[e] = ra;
    b[e] = rb;
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if constexpr (EB == 4) {
      lo[w] = __float_as_uint(a[w]);
      hi[w] = __float_as_uint(b[w]);
    } else {
      lo[w] = Tag::pack2(a[2 * w], a[2 * w + 1]);
      hi[w] = Tag::pack2(b[2 * w], b[2 * w + 1]);
    }
  }
}

}  // namespace attn
