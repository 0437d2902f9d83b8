// Internal launchers shared between translation units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Advance of a static append cache's lengths, kv_len[b] = min(kv_len[b] + T,
// cap) for b < B, done by a kernel that runs after every reader of kv_len in
// the same step (kv_len null: none)
struct KvAdvance {
  int* kv_len = nullptr;
  int B = 0, T = 0, cap = 0;
};

// Merge split partials o_part [R, nsplit, D] / lse_part [R, nsplit] into
// o [R, D] (out_dtype) on `stream`; lse_out [R] (natural log), if given,
// receives the merged log-sum-exp.
// The combine also applies `adv` (first workgroup), when given.
void launch_combine(const float* o_part, const float* lse_part, void* o, int R, int nsplit, int D,
                    int out_dtype, hipStream_t stream, float* lse_out = nullptr, KvAdvance adv = {});

// The same with the partial outputs stored as bf16 bits (o_part [R, nsplit, D]).
void launch_combine_bf16_parts(const uint16_t* o_part, const float* lse_part, void* o, int R, int nsplit,
                               int D, int out_dtype, hipStream_t stream, float* lse_out = nullptr,
                               KvAdvance adv = {});

// kv_len[b] = min(kv_len[b] + T, cap) as a launch of its own
void launch_kv_advance(const KvAdvance& adv, hipStream_t stream);

// Workspace layout of the decode calls: partial outputs first, then the
// partial log-sum-exps, each 256-byte aligned.
struct SplitWorkspace {
  size_t o_bytes;
  size_t lse_offset;
  size_t total;
};

inline SplitWorkspace split_workspace(long long rows, long long nsplit, long long d, int part_bytes = 4) {
  SplitWorkspace w;
  w.o_bytes = (size_t)(rows * nsplit * d) * part_bytes;
  w.lse_offset = (w.o_bytes + 255) / 256 * 256;
  w.total = w.lse_offset + ((size_t)(rows * nsplit) * sizeof(float) + 255) / 256 * 256;
  return w;
}

}  // namespace attn
