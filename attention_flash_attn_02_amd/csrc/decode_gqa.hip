// Split-context GQA decode ("flash-decoding") against a static KV cache.
//
// Follows the fixed-budget decode audit (sections "Which implementation was
// tested" and "Setup and interpretation"): one new query token per sequence,
// a static append cache (capacity 2056 for a 2048 context), the context cut
// into splits of 128 slots, and the G query heads of a KV head grouped so one
// pass over a K/V tile serves all of them (the audit notes that such a row
// tile carries few useful query rows; here they ride in the 16-wide N side
// of a 16x16x32 MFMA).
//
// Kernel 1 (this file): one workgroup per (split, KV head, sequence); each
// wave takes 32-slot chunks of the split:
//   * K rows go straight from HBM into registers as the A operand of
//     S^T = K Q^T (16 B per lane per load, whole 256-B rows per 16 lanes);
//   * V rows are loaded with whole-row coalescing, transposed in registers
//     and written to the wave's own LDS area as V^T, whose slot order inside
//     each 32-slot chunk matches the score accumulator, so O^T += V^T P^T
//     takes its A operand as one 16-byte LDS read;
//   * per-wave online softmax; the waves' partials are merged through LDS and
//     one (o, lse) partial per query head and split is written to the
//     workspace.
// Kernel 2 (combine.hip) merges the splits.
// Slots at or past kv_len are never loaded; a split that starts past kv_len
// writes the empty partial (o = 0, lse = -inf).

#include "common.hpp"
#include "kernels.hpp"

namespace attn {

struct DecodeGqaParams {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* kv_len;
  float* o_part;
  float* lse_part;
  int Hq, Hkv, G, cap, split, nsplit;
  float scale_log2;
};

template <class Tag, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void decode_gqa_split_kernel(const DecodeGqaParams p) {
  constexpr int D = 128;
  constexpr int NDB = D / 16;  // 16-row blocks of O^T
  constexpr int NKK = D / 32;  // 32-wide k-steps of S^T
  constexpr int VP = 32 + 8;   // V^T row pitch in 16-bit elements
  __shared__ __attribute__((aligned(16))) uint16_t vt[WAVES][D * VP];
  __shared__ float red_m[WAVES][16];
  __shared__ float red_l[WAVES][16];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m16 = lane & 15, qq = lane >> 4;
  const int split_idx = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int L = min(max(p.kv_len[b], 0), p.cap);
  const int s0 = split_idx * p.split;
  const int s1 = min(s0 + p.split, L);
  const int row0 = b * p.Hq + kvh * p.G;  // first output row (query head) of this KV head

  if (s0 >= s1) {  // empty split
    for (int idx = tid; idx < p.G * D; idx += WAVES * 64)
      p.o_part[((size_t)(row0 + idx / D) * p.nsplit + split_idx) * D + idx % D] = 0.f;
    if (tid < p.G) p.lse_part[(size_t)(row0 + tid) * p.nsplit + split_idx] = kNegInf;
    return;
  }

  // query fragments: B operand of S^T (columns m < G are real heads)
  u32x4 qf[NKK];
  {
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(p.q) + ((size_t)(row0 + m16) * D) * 2;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = m16 < p.G ? ldg16(qrow + (32 * kk + 8 * qq) * 2) : u32x4{0, 0, 0, 0};
  }

  const size_t kv_base = ((size_t)b * p.Hkv + kvh) * p.cap;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.kc) + kv_base * D * 2;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.vc) + kv_base * D * 2;
  uint16_t* vtw = vt[wave];
  const int vdc = lane & 15, vtg = lane >> 4;  // V staging: d chunk, token group of 8
  const int vpos = 16 * (vtg & 1) + 4 * (vtg >> 1);

  f32x4 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  for (int c0 = s0 + 32 * wave; c0 < s1; c0 += 32 * WAVES) {
    u32x4 kf[2][NKK];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int tok = c0 + 16 * tb + m16;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        kf[tb][kk] = tok < s1 ? ldg16(kbase + ((size_t)tok * D + 32 * kk + 8 * qq) * 2) : u32x4{0, 0, 0, 0};
    }
    u32x4 vr[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int tok = c0 + 8 * vtg + r;
      vr[r] = tok < s1 ? ldg16(vbase + ((size_t)tok * D + 8 * vdc) * 2) : u32x4{0, 0, 0, 0};
    }

    // S^T = K Q^T: lane holds slots 16 tb + 4 qq + i for query column m16
    f32x4 sacc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      sacc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) sacc[tb] = Tag::mfma16(kf[tb][kk], qf[kk], sacc[tb]);
    }

    // V^T for this chunk -> this wave's LDS area
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = i >> 1;
      uint16_t* dst = vtw + (8 * vdc + i) * VP + vpos;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 a0 = vr[4 * h], a1 = vr[4 * h + 1], a2 = vr[4 * h + 2], a3 = vr[4 * h + 3];
        u32x2 o;
        o[0] = (i & 1) ? ((a0[e] >> 16) | (a1[e] & 0xffff0000u)) : ((a0[e] & 0xffffu) | (a1[e] << 16));
        o[1] = (i & 1) ? ((a2[e] >> 16) | (a3[e] & 0xffff0000u)) : ((a2[e] & 0xffffu) | (a3[e] << 16));
        *reinterpret_cast<u32x2*>(dst + 8 * h) = o;
      }
    }

    // online softmax over the chunk's 32 slots
    float s[8];
    float mx = kNegInf;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = c0 + 16 * tb + 4 * qq + i;
        const float x = tok < s1 ? sacc[tb][i] * p.scale_log2 : kNegInf;
        s[4 * tb + i] = x;
        mx = fmaxf(mx, x);
      }
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m_run, mx);  // finite: every chunk holds a valid slot
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float pv[8], psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pv[j] = fast_exp2(s[j] - m_new);
      psum += pv[j];
    }
    l_run = l_run * alpha + psum;
    const u32x4 pf = {Tag::pack2(pv[0], pv[1]), Tag::pack2(pv[2], pv[3]), Tag::pack2(pv[4], pv[5]),
                      Tag::pack2(pv[6], pv[7])};
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      acc_o[db] *= alpha;
      const u32x4 a = *reinterpret_cast<const u32x4*>(vtw + (16 * db + m16) * VP + 8 * qq);
      acc_o[db] = Tag::mfma16(a, pf, acc_o[db]);
    }
  }

  // ---- merge the waves' partials ----
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  float* ow = reinterpret_cast<float*>(vtw);  // reuse this wave's V^T area: [16][D] floats
  if (m16 < p.G) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) ow[m16 * D + 16 * db + 4 * qq + i] = acc_o[db][i];
    if (qq == 0) {
      red_m[wave][m16] = m_run;
      red_l[wave][m16] = l_run;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < p.G * D; idx += WAVES * 64) {
    const int mm = idx / D, d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, red_m[w][mm]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float f = fast_exp2(red_m[w][mm] - M);
      o = fmaf(f, reinterpret_cast<const float*>(vt[w])[mm * D + d], o);
      l = fmaf(f, red_l[w][mm], l);
    }
    const size_t prow = (size_t)(row0 + mm) * p.nsplit + split_idx;
    p.o_part[prow * D + d] = o / l;
    if (d == 0) p.lse_part[prow] = (M + __log2f(l)) * kLn2;
  }
}

template <class Tag>
static void launch_split(const DecodeGqaParams& p, int waves, dim3 grid, hipStream_t st) {
  if (waves == 4) hipLaunchKernelGGL((decode_gqa_split_kernel<Tag, 4>), grid, dim3(256), 0, st, p);
  else if (waves == 2) hipLaunchKernelGGL((decode_gqa_split_kernel<Tag, 2>), grid, dim3(128), 0, st, p);
  else hipLaunchKernelGGL((decode_gqa_split_kernel<Tag, 1>), grid, dim3(64), 0, st, p);
}

}  // namespace attn

using namespace attn;

static const int kDefaultGqaSplit = 128;

static int gqa_split(int split) { return split <= 0 ? kDefaultGqaSplit : split; }

extern "C" size_t attn_decode_gqa_workspace_bytes(int B, int Hq, int cap, int D, int split) {
  split = gqa_split(split);
  if (B <= 0 || Hq <= 0 || cap <= 0 || D <= 0 || split <= 0) return 0;
  const long long nsplit = (cap + split - 1) / split;
  return split_workspace((long long)B * Hq, nsplit, D).total;
}

extern "C" attn_status attn_decode_gqa(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* kv_len, void* o, void* workspace,
                                       size_t workspace_bytes, int B, int Hq, int Hkv, int D,
                                       int cap, int split, attn_dtype dtype, float softmax_scale,
                                       hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !kv_len || !o) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || cap <= 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_BF16 && dtype != ATTN_F16) {
    if (dtype < ATTN_F32 || dtype > ATTN_FP8_E5M2) return ATTN_ERR_DTYPE;
    return ATTN_ERR_UNSUPPORTED;
  }
  if (D != 128 || Hq / Hkv > 16) return ATTN_ERR_UNSUPPORTED;
  split = gqa_split(split);
  if (split % 32 != 0 || split < 32 || split > 1024) return ATTN_ERR_SHAPE;
  if (B > 65535 || Hkv > 65535) return ATTN_ERR_SHAPE;
  if (!(softmax_scale == softmax_scale)) return ATTN_ERR_SHAPE;
  if (!attn_host::aligned(q, 16) || !attn_host::aligned(k_cache, 16) ||
      !attn_host::aligned(v_cache, 16) || !attn_host::aligned(o, 16) ||
      !attn_host::aligned(kv_len, 4))
    return ATTN_ERR_ALIGN;
  const int nsplit = (cap + split - 1) / split;
  const SplitWorkspace ws = split_workspace((long long)B * Hq, nsplit, D);
  if (!workspace || workspace_bytes < ws.total) return ATTN_ERR_WORKSPACE;
  if (!attn_host::aligned(workspace, 256)) return ATTN_ERR_ALIGN;

  DecodeGqaParams p{};
  p.q = q; p.kc = k_cache; p.vc = v_cache; p.kv_len = kv_len;
  p.o_part = reinterpret_cast<float*>(workspace);
  p.lse_part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + ws.lse_offset);
  p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.cap = cap; p.split = split; p.nsplit = nsplit;
  p.scale_log2 = softmax_scale * kLog2e;
  const int waves = split >= 128 ? 4 : split / 32;
  dim3 grid(nsplit, Hkv, B);
  if (dtype == ATTN_BF16) launch_split<Bf16Tag>(p, waves, grid, stream);
  else launch_split<F16Tag>(p, waves, grid, stream);
  attn_status st = attn_host::launch_status();
  if (st != ATTN_OK) return st;
  launch_combine(p.o_part, p.lse_part, o, B * Hq, nsplit, D, dtype, stream);
  return attn_host::launch_status();
}
