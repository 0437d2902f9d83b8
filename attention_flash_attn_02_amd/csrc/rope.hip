// Standalone rotary position embedding: the unfused form of the prefill's
// RoPE step.  The shape-adaptive attention lesson page (rows "What was tried"
// and "Actual result") compares RoPE fused into the attention kernel with
// RoPE as separate kernels; this kernel rotates Q or K in HBM so that the
// attention kernel can run without RoPE.
//
// Operation (rotate-half): for row (b, h, s) at position s, the pair
// (x[i], x[i + D/2]) becomes (x[i] cos a - x[i+D/2] sin a,
// x[i+D/2] cos a + x[i] sin a) with a = s * theta^(-2i/D), in fp32 with the
// angle reduced to one revolution from an exact three-part split of the
// frequency; the result is rounded once to the element type (round to
// nearest even).
//
// One thread per row and 16-byte chunk of the first half: it loads the
// chunk and its partner chunk D/2 elements later, rotates the pairs and
// stores both, so the rotation is done in place when y == x (every element
// is read and written by the same thread).

#include "common.hpp"

namespace attn {

struct RopeParams {
  const void* x;
  void* y;
  long long rows;  // B * H * S
  int S, D;
  float rope_fhi[128];
  float rope_fmid[128];
  float rope_flo[128];
};

struct F32Elem {
  static constexpr int kBytes = 4;
};

template <class Tag>
__global__ __launch_bounds__(256) void rope_kernel(const RopeParams p) {
  constexpr int EB = Tag::kBytes;
  constexpr int EPC = 16 / EB;  // elements per 16-byte chunk
  const int half = p.D / 2;
  const int cpr = half / EPC;  // chunks per half row
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= p.rows * cpr) return;
  const long long row = t / cpr;
  const int c = (int)(t % cpr);
  const float pos = (float)(int)(row % p.S);
  const uint8_t* xr = reinterpret_cast<const uint8_t*>(p.x) + row * p.D * EB;
  uint8_t* yr = reinterpret_cast<uint8_t*>(p.y) + row * p.D * EB;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(xr + 16 * c);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(xr + half * EB + 16 * c);
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
    const float rev = __builtin_amdgcn_fractf(__builtin_amdgcn_fractf(pos * p.rope_fhi[i]) +
                                              __builtin_amdgcn_fractf(pos * p.rope_fmid[i]) + pos * p.rope_flo[i]);
    const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
    const float ra = a[e] * cs - b[e] * sn, rb = b[e] * cs + a[e] * sn;
    a[e] = ra;
    b[e] = rb;
  }
  u32x4 olo, ohi;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if constexpr (EB == 4) {
      olo[w] = __float_as_uint(a[w]);
      ohi[w] = __float_as_uint(b[w]);
    } else {
      olo[w] = Tag::pack2(a[2 * w], a[2 * w + 1]);
      ohi[w] = Tag::pack2(b[2 * w], b[2 * w + 1]);
    }
  }
  *reinterpret_cast<u32x4*>(yr + 16 * c) = olo;
  *reinterpret_cast<u32x4*>(yr + half * EB + 16 * c) = ohi;
}

}  // namespace attn

using namespace attn;

extern "C" attn_status attn_rope_rotate(const void* x, void* y, int B, int H, int S, int D, attn_dtype dtype,
                                        float rope_theta, hipStream_t stream) {
  if (!x || !y) return ATTN_ERR_NULL;
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0 || D % 2 != 0) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) {
    if (dtype == ATTN_FP8_E5M2) return ATTN_ERR_UNSUPPORTED;
    return ATTN_ERR_DTYPE;
  }
  if (!(rope_theta > 0.f) || !(rope_theta < 3.0e38f)) return ATTN_ERR_SHAPE;
  const int eb = dtype == ATTN_F32 ? 4 : 2;
  // whole 16-byte chunks in each half row; at most 256 dims
  if (D > 256 || ((D / 2) * eb) % 16 != 0) return ATTN_ERR_UNSUPPORTED;
  if (S > 65536) return ATTN_ERR_UNSUPPORTED;  // exact angle reduction needs pos < 2^16
  if (!attn_host::aligned(x, 16) || !attn_host::aligned(y, 16)) return ATTN_ERR_ALIGN;
  const long long rows = (long long)B * H * S;
  const long long threads = rows * ((D / 2) * eb / 16);
  if ((threads + 255) / 256 > 0x7fffffffLL) return ATTN_ERR_SHAPE;

  RopeParams p{};
  p.x = x; p.y = y; p.rows = rows; p.S = S; p.D = D;
  attn_host::rope_freq_split(rope_theta, D, nullptr, p.rope_fhi, p.rope_flo, p.rope_fmid);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (dtype == ATTN_BF16) hipLaunchKernelGGL((rope_kernel<Bf16Tag>), grid, block, 0, stream, p);
  else if (dtype == ATTN_F16) hipLaunchKernelGGL((rope_kernel<F16Tag>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((rope_kernel<F32Elem>), grid, block, 0, stream, p);
  return attn_host::launch_status();
}
