// Parameters and small device helpers shared by the prefill kernels.
#pragma once

#include "common.hpp"

namespace attn {

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, S;
  int D;          // head dim
  int G;          // Hq / Hkv
  int GP;         // heads of one KV group handled by one workgroup
  int P;          // query positions per workgroup
  int n_ptiles;   // ceil(S / P)
  int n_hgroups;  // G / GP
  float scale_log2;  // softmax_scale * q_descale * k_descale * log2(e)
  float out_scale;   // v_descale
  int out_dtype;
  int rope;
  float inv_freq[64];  // RoPE inverse frequencies theta^(-2i/D), i < D/2
  // RoPE frequencies in revolutions per position, f = theta^(-2i/D) / (2 pi),
  // split as f_hi + f_lo with f_hi carrying 8 significant bits: pos * f_hi is
  // then exact in fp32 for pos < 2^16, so frac(pos * f_hi) + pos * f_lo gives
  // the angle modulo one revolution to ~1e-7 without fp64 arithmetic.
  float rope_fhi[64];
  float rope_flo[64];
  float rope_fmid[64];  // three-way split (f_hi + f_mid + f_lo) for the fp32 kernel
  int halves;  // MFMA kernel: 1 = 4-wave workgroups, 2 = 8-wave split-key workgroups
  int persist;  // 4-wave kernel with resident workgroups looping over items (grid < items)
  int pingpong;  // 8-wave kernel: the two halves run half a key tile apart (see PP)
  int regstage;  // 4-wave kernel: K and V tiles staged through registers (see RS)
  // chunked prefill against a cache prefix (prefill_fwd_kernel<..., CHUNK>)
  const int* kv_len;  // [B] key lengths (with kv_add: the chunk's tokens), device memory
  int kv_add;         // added to kv_len[b]: 0, or the chunk length when kv_len excludes the chunk
  // chunk mode that appends the chunk itself (k_new non-null): the chunk's
  // keys and values [B, Hkv, S, D], written by the kernel to the cache rows
  // kv_len[b] + t (K rotated there with the three-part frequency split
  // rope_fhi / rope_fmid / rope_flo3, as the append kernel does)
  const void* k_new;
  const void* v_new;
  float rope_flo3[64];
  int cap;            // cache slots per head
  int nsplit;         // key ranges per item (1: results go straight to o / lse)
  int split_keys;     // keys per range, a multiple of 64
  float* ws_o;        // [B*Hq*S, nsplit, D] partial outputs (nsplit > 1; bf16 bits in chunk mode)
  float* ws_lse;      // [B*Hq*S, nsplit] partial log-sum-exps (nsplit > 1)
};

typedef __attribute__((ext_vector_type(4))) short v4i16;
#define LDS_AS(T, ptr) ((__attribute__((address_space(3))) T*)(ptr))

// max / sum of x over lanes l and l ^ 32: v_permlane32_swap of x with itself
// leaves one copy of x and one copy of the partner's x in the two results.
__device__ inline float pair_max32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (gfx9 encoding: vmcnt bits [3:0] and [15:14];
// expcnt and lgkmcnt left at their maxima, i.e. not waited for)
// software-pipelined 16-bit prefill kernel (one wave per SIMD), prefill_sp.hip
// (halves 1: 4-wave workgroups; 2: 8-wave workgroups splitting the key tiles)
void launch_prefill_sp(const PrefillParams& p, bool bf16, bool causal, bool rope_q, int halves, hipStream_t st);
// software-pipelined fp8 e5m2 prefill kernel (P in e4m3), prefill_sp8.hip
void launch_prefill_sp8(const PrefillParams& p, bool causal, hipStream_t st);

constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

}  // namespace attn
