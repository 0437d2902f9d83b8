// Split-softmax combine: merge per-split partial attention results.
//
// Each split s of a row carries its output normalised within the split,
// o_s, and the natural-log log-sum-exp of its scaled scores, lse_s.  The
// merged row is sum_s w_s o_s / sum_s w_s with w_s = exp(lse_s - max lse).
// Folding two parts at a time with alpha = sigmoid(lse_b - lse_a),
// o = (1 - alpha) o_a + alpha o_b (the merge rule of the fixed-budget
// decode audit, section "A: group-entry queries and one joint history
// scan") reaches the same result; the weighted sum does it in one pass.
// Empty splits (lse = -inf) have weight 0; a row whose splits are all
// empty is written as zeros.

#include "common.hpp"
#include "kernels.hpp"

namespace attn {

// the cache-length advance a combine can carry (before any early exit: the
// combine never reads kv_len, and every kernel that did has finished)
__device__ inline void kv_advance(const KvAdvance& a) {
  if (a.kv_len && blockIdx.x == 0)
    for (int i = threadIdx.x; i < a.B; i += blockDim.x) a.kv_len[i] = min(max(a.kv_len[i], 0) + a.T, a.cap);
}

// One thread per (row, 4 consecutive dims): every thread recomputes the
// row's split weights from the (cached) lse values and then reads its float4
// of every split with independent loads.  Requires D % 4 == 0.
__global__ __launch_bounds__(256) void combine_kernel_v4(const float* __restrict__ o_part,
                                                         const float* __restrict__ lse_part,
                                                         void* __restrict__ o, float* __restrict__ lse_out,
                                                         int R, int nsplit, int D, int out_dtype, KvAdvance adv) {
  kv_advance(adv);
  const int d4n = D >> 2;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)R * d4n) return;
  const int r = (int)(t / d4n), d = 4 * (int)(t % d4n);
  const float* lse = lse_part + (size_t)r * nsplit;
  float mx = kNegInf;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, lse[s]);
  const size_t oidx = (size_t)r * D + d;
  if (mx == kNegInf) {
    store4(o, oidx, out_dtype, 0.f, 0.f, 0.f, 0.f);
    if (lse_out && d == 0) lse_out[r] = kNegInf;
    return;
  }
  const f32x4* op = reinterpret_cast<const f32x4*>(o_part + (size_t)r * nsplit * D + d);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  int s = 0;
  for (; s + 4 <= nsplit; s += 4) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = op[(size_t)(s + u) * d4n];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = fast_exp2((lse[s + u] - mx) * kLog2e);
      wsum += w;
      acc += w * v[u];
    }
  }
  for (; s < nsplit; ++s) {
    const float w = fast_exp2((lse[s] - mx) * kLog2e);
    wsum += w;
    acc += w * op[(size_t)s * d4n];
  }
  const float inv = 1.f / wsum;
  store4(o, oidx, out_dtype, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  if (lse_out && d == 0) lse_out[r] = mx + __log2f(wsum) * kLn2;
}

// The same for at most NS parts: every lse and every float4 of the row's
// parts is loaded up front, which leaves one memory round trip per thread
// instead of one per group of parts.  The buffer descriptors cover the whole
// part and lse arrays (the same for every lane, so the loads take them as
// they are): a load for a split s >= nsplit reads the next row's values,
// which get weight 0, or, past the last row, zero without a memory access.
template <int NS>
__global__ __launch_bounds__(256) void combine_kernel_v4s(const float* __restrict__ o_part,
                                                          const float* __restrict__ lse_part,
                                                          void* __restrict__ o, float* __restrict__ lse_out,
                                                          int R, int nsplit, int D, int out_dtype, KvAdvance adv) {
  kv_advance(adv);
  const int d4n = D >> 2;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)R * d4n) return;
  const int r = (int)(t / d4n), d = 4 * (int)(t % d4n);
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(lse_part), (short)0, R * nsplit * 4, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t ors =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(o_part), (short)0, R * nsplit * D * 4, kBufferRsrcWord3);
  const int l0 = 4 * r * nsplit, o0 = 4 * (r * nsplit * D + d);  // byte offsets of split 0
  float l[NS];
  f32x4 v[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    l[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, l0 + 4 * s, 0, 0));
    v[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ors, o0 + 4 * s * D, 0, 0));
  }
  float mx = kNegInf;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < nsplit) mx = fmaxf(mx, l[s]);
  const size_t oidx = (size_t)r * D + d;
  if (mx == kNegInf) {
    store4(o, oidx, out_dtype, 0.f, 0.f, 0.f, 0.f);
    if (lse_out && d == 0) lse_out[r] = kNegInf;
    return;
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s < nsplit) {  // (a uniform branch: loads past the row read other rows' values, never used)
      const float w = fast_exp2((l[s] - mx) * kLog2e);
      wsum += w;
      acc += w * v[s];
    }
  }
  const float inv = 1.f / wsum;
  store4(o, oidx, out_dtype, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  if (lse_out && d == 0) lse_out[r] = mx + __log2f(wsum) * kLn2;
}

// Parts stored as bf16 bits (half the bytes of fp32 parts; used by the MLA
// decode, whose parts are 448 wide, and by chunked prefill): one thread per
// (row, 4 dims), the loop of combine_kernel_v4 over 8-byte loads; optional
// merged LSE and kv_len advance as in combine_kernel_v4.
__global__ __launch_bounds__(256) void combine_kernel_v4_bf16(const uint16_t* __restrict__ o_part,
                                                              const float* __restrict__ lse_part,
                                                              void* __restrict__ o, float* __restrict__ lse_out,
                                                              int R, int nsplit, int D, int out_dtype,
                                                              KvAdvance adv) {
  kv_advance(adv);
  const int d4n = D >> 2;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)R * d4n) return;
  const int r = (int)(t / d4n), d = 4 * (int)(t % d4n);
  const float* lse = lse_part + (size_t)r * nsplit;
  float mx = kNegInf;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, lse[s]);
  const size_t oidx = (size_t)r * D + d;
  if (mx == kNegInf) {
    store4(o, oidx, out_dtype, 0.f, 0.f, 0.f, 0.f);
    if (lse_out && d == 0) lse_out[r] = kNegInf;
    return;
  }
  const u32x2* op = reinterpret_cast<const u32x2*>(o_part + (size_t)r * nsplit * D + d);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  int s = 0;
  for (; s + 4 <= nsplit; s += 4) {
    u32x2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = op[(size_t)(s + u) * d4n];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = fast_exp2((lse[s + u] - mx) * kLog2e);
      wsum += w;
      acc += w * f32x4{Bf16Tag::to_f32(v[u][0] & 0xffff), Bf16Tag::to_f32(v[u][0] >> 16),
                       Bf16Tag::to_f32(v[u][1] & 0xffff), Bf16Tag::to_f32(v[u][1] >> 16)};
    }
  }
  for (; s < nsplit; ++s) {
    const u32x2 v = op[(size_t)s * d4n];
    const float w = fast_exp2((lse[s] - mx) * kLog2e);
    wsum += w;
    acc += w * f32x4{Bf16Tag::to_f32(v[0] & 0xffff), Bf16Tag::to_f32(v[0] >> 16), Bf16Tag::to_f32(v[1] & 0xffff),
                     Bf16Tag::to_f32(v[1] >> 16)};
  }
  const float inv = 1.f / wsum;
  store4(o, oidx, out_dtype, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  if (lse_out && d == 0) lse_out[r] = mx + __log2f(wsum) * kLn2;
}

void launch_combine_bf16_parts(const uint16_t* o_part, const float* lse_part, void* o, int R, int nsplit,
                               int D, int out_dtype, hipStream_t stream, float* lse_out, KvAdvance adv) {
  const long long threads = (long long)R * (D / 4);
  hipLaunchKernelGGL(combine_kernel_v4_bf16, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, o_part,
                     lse_part, o, lse_out, R, nsplit, D, out_dtype, adv);
}

// General D: one wave per row, four rows per workgroup.  Lane s holds split
// s's weight (splits beyond 64 are folded in a loop), the weights are
// broadcast with readlane, and the partial rows are read with independent
// loads.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      void* __restrict__ o, float* __restrict__ lse_out,
                                                      int R, int nsplit, int D, int out_dtype, KvAdvance adv) {
  kv_advance(adv);
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= R) return;
  const float* lse = lse_part + (size_t)r * nsplit;
  float mx = kNegInf;
  for (int s = lane; s < nsplit; s += 64) mx = fmaxf(mx, lse[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const size_t obase = (size_t)r * D;
  if (mx == kNegInf) {
    for (int d = lane; d < D; d += 64) store1(o, obase + d, out_dtype, 0.f);
    if (lse_out && lane == 0) lse_out[r] = kNegInf;
    return;
  }
  float wsum = 0.f;
  for (int s = lane; s < nsplit; s += 64) wsum += fast_exp2((lse[s] - mx) * kLog2e);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
  const float inv = 1.f / wsum;
  if (lse_out && lane == 0) lse_out[r] = mx + __log2f(wsum) * kLn2;
  const float* op = o_part + (size_t)r * nsplit * D;
  for (int d0 = 0; d0 < D; d0 += 64) {
    const int d = d0 + lane;
    float acc = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 64) {
      const float w_l = s0 + lane < nsplit ? fast_exp2((lse[s0 + lane] - mx) * kLog2e) : 0.f;
      const int ns = min(64, nsplit - s0);
      int s = 0;
      for (; s + 4 <= ns; s += 4) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = d < D ? op[(size_t)(s0 + s + u) * D + d] : 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = fmaf(__shfl(w_l, s + u), v[u], acc);
      }
      for (; s < ns; ++s) {
        const float v = d < D ? op[(size_t)(s0 + s) * D + d] : 0.f;
        acc = fmaf(__shfl(w_l, s), v, acc);
      }
    }
    if (d < D) store1(o, obase + d, out_dtype, acc * inv);
  }
}

void launch_combine(const float* o_part, const float* lse_part, void* o, int R, int nsplit, int D,
                    int out_dtype, hipStream_t stream, float* lse_out, KvAdvance adv) {
  if (D % 4 == 0) {
    const long long threads = (long long)R * (D / 4);
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    // (buffer ranges and offsets are 32-bit: all parts, plus the loads past
    // the last row's, must span less than 2 GiB)
    // up to 8 parts: every load up front (GQA decode's five parts: 5.1 -> 4.7 us
    // at batch 128); more parts: the loop (loading 16 slots for MLA's nine
    // parts was slower, 8.9 vs 7.6 us)
    if (nsplit <= 8 && ((long long)R * nsplit + 8) * D * 4 < (1LL << 31))
      hipLaunchKernelGGL(combine_kernel_v4s<8>, grid, block, 0, stream, o_part, lse_part, o, lse_out, R, nsplit, D,
                         out_dtype, adv);
    else
      hipLaunchKernelGGL(combine_kernel_v4, grid, block, 0, stream, o_part, lse_part, o, lse_out, R, nsplit, D,
                         out_dtype, adv);
  } else {
    hipLaunchKernelGGL(combine_kernel, dim3((R + 3) / 4), dim3(256), 0, stream, o_part, lse_part, o, lse_out,
                       R, nsplit, D, out_dtype, adv);
  }
}

}  // namespace attn

extern "C" attn_status attn_combine_splits(const float* o_part, const float* lse_part, void* o,
                                           int R, int nsplit, int D, attn_dtype out_dtype,
                                           hipStream_t stream) {
  if (!o_part || !lse_part || !o) return ATTN_ERR_NULL;
  if (R <= 0 || nsplit <= 0 || D <= 0 || D > 1024) return ATTN_ERR_SHAPE;
  if (out_dtype != ATTN_F32 && out_dtype != ATTN_F16 && out_dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (!attn_host::aligned(o_part, 4) || !attn_host::aligned(lse_part, 4) ||
      !attn_host::aligned(o, out_dtype == ATTN_F32 ? 4 : 2))
    return ATTN_ERR_ALIGN;
  attn::launch_combine(o_part, lse_part, o, R, nsplit, D, out_dtype, stream);
  return attn_host::launch_status();
}

extern "C" const char* attn_status_str(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer argument";
    case ATTN_ERR_SHAPE: return "invalid or inconsistent shape";
    case ATTN_ERR_DTYPE: return "unsupported dtype";
    case ATTN_ERR_ALIGN: return "misaligned pointer";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}
