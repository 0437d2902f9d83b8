// Absorbed-MLA decode against a latent cache (448-d latent + 64-d RoPE per
// token), split over the context and merged by the combine kernel.
//
// The fixed-budget decode audit ("Which implementation was tested") runs MLA
// with a 448-d latent plus 64-d RoPE key per token and matrix absorption in
// eager PyTorch, and notes that no optimized MLA decode kernel exists in that
// project.  With absorption the H query heads all attend to the same cache
// rows: scores use the full 512-d row and values are its 448-d latent part,
// so one pass over the cache serves all heads (16 heads fill the 16-wide N
// side of a 16x16x32 MFMA).
//
// One workgroup (4 waves) per (split, sequence).  For each 32-slot chunk:
//   * the 32 cache rows (32 KB) are staged once in LDS with full-row
//     coalesced loads (prefetched into registers during the previous chunk);
//   * every wave computes the same S^T = C Q^T (32 x 16) from LDS, so the
//     online-softmax state is identical in all waves without any exchange;
//   * each wave then owns 7 of the 28 16-row blocks of O^T = C_lat^T P^T and
//     reads its A operand (cache rows transposed) from LDS.
// Slots at or past kv_len are never loaded; a split that starts past kv_len
// writes the empty partial (o = 0, lse = -inf).

#include "common.hpp"
#include "kernels.hpp"

namespace attn {

struct DecodeMlaParams {
  const void* q;
  const void* c;
  const int32_t* kv_len;
  float* o_part;
  float* lse_part;
  int H, cap, split, nsplit;
  float scale_log2;
};

template <class Tag>
__global__ __launch_bounds__(256) void decode_mla_split_kernel(const DecodeMlaParams p) {
  constexpr int DQ = 512, DL = 448;
  constexpr int CP = DQ + 8;         // LDS row pitch (16-bit elements)
  constexpr int NKK = DQ / 32;       // 32-wide k-steps of S^T
  constexpr int DBW = DL / 16 / 4;   // 16-row O^T blocks per wave (7)
  __shared__ __attribute__((aligned(16))) uint16_t cl[32 * CP];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m16 = lane & 15, qq = lane >> 4;
  const int split_idx = blockIdx.x, b = blockIdx.y;
  const int L = min(max(p.kv_len[b], 0), p.cap);
  const int s0 = split_idx * p.split;
  const int s1 = min(s0 + p.split, L);
  const int row0 = b * p.H;

  if (s0 >= s1) {  // empty split
    for (int idx = tid; idx < p.H * DL; idx += 256)
      p.o_part[((size_t)(row0 + idx / DL) * p.nsplit + split_idx) * DL + idx % DL] = 0.f;
    if (tid < p.H) p.lse_part[(size_t)(row0 + tid) * p.nsplit + split_idx] = kNegInf;
    return;
  }

  u32x4 qf[NKK];
  {
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(p.q) + ((size_t)(row0 + m16) * DQ) * 2;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = m16 < p.H ? ldg16(qrow + (32 * kk + 8 * qq) * 2) : u32x4{0, 0, 0, 0};
  }

  const uint8_t* cbase = reinterpret_cast<const uint8_t*>(p.c) + ((size_t)b * p.cap) * DQ * 2;
  const int srow = tid >> 6, scol = tid & 63;  // staging: rows srow + 4u, 16-B column scol
  u32x4 cb[8];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int tok = c0 + srow + 4 * u;
      cb[u] = tok < s1 ? ldg16(cbase + ((size_t)tok * DQ + 8 * scol) * 2) : u32x4{0, 0, 0, 0};
    }
  };

  f32x4 acc_o[DBW];
#pragma unroll
  for (int i = 0; i < DBW; ++i) acc_o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  load_chunk(s0);
  for (int c0 = s0; c0 < s1; c0 += 32) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) *reinterpret_cast<u32x4*>(cl + (srow + 4 * u) * CP + 8 * scol) = cb[u];
    if (c0 + 32 < s1) load_chunk(c0 + 32);
    __syncthreads();

    f32x4 sacc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      sacc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* crow = cl + (16 * tb + m16) * CP + 8 * qq;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        sacc[tb] = Tag::mfma16(*reinterpret_cast<const u32x4*>(crow + 32 * kk), qf[kk], sacc[tb]);
    }

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
    const float m_new = fmaxf(m_run, mx);
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

    // O^T rows d = 16 db + ..., A operand slot j <-> chunk slot 16 (j/4) + 4 qq + j%4
#pragma unroll
    for (int i = 0; i < DBW; ++i) {
      const int d = 16 * (wave * DBW + i) + m16;
      uint32_t a[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j0 = 2 * e, j1 = 2 * e + 1;
        const uint32_t lo = cl[(16 * (j0 >> 2) + 4 * qq + (j0 & 3)) * CP + d];
        const uint32_t hi = cl[(16 * (j1 >> 2) + 4 * qq + (j1 & 3)) * CP + d];
        a[e] = lo | (hi << 16);
      }
      acc_o[i] *= alpha;
      acc_o[i] = Tag::mfma16(u32x4{a[0], a[1], a[2], a[3]}, pf, acc_o[i]);
    }
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (m16 < p.H) {
    const float inv = 1.f / l_run;
    const size_t prow = (size_t)(row0 + m16) * p.nsplit + split_idx;
#pragma unroll
    for (int i = 0; i < DBW; ++i) {
      const int d = 16 * (wave * DBW + i) + 4 * qq;
      *reinterpret_cast<f32x4*>(p.o_part + prow * DL + d) = acc_o[i] * inv;
    }
    if (wave == 0 && qq == 0) p.lse_part[prow] = (m_run + __log2f(l_run)) * kLn2;
  }
}

}  // namespace attn

using namespace attn;

static const int kDefaultMlaSplit = 256;

static int mla_split(int split) { return split <= 0 ? kDefaultMlaSplit : split; }

extern "C" size_t attn_decode_mla_workspace_bytes(int B, int H, int cap, int d_latent, int split) {
  split = mla_split(split);
  if (B <= 0 || H <= 0 || cap <= 0 || d_latent <= 0 || split <= 0) return 0;
  const long long nsplit = (cap + split - 1) / split;
  return split_workspace((long long)B * H, nsplit, d_latent).total;
}

extern "C" attn_status attn_decode_mla(const void* q, const void* kv_cache, const int32_t* kv_len,
                                       void* o, void* workspace, size_t workspace_bytes, int B,
                                       int H, int d_latent, int d_rope, int cap, int split,
                                       attn_dtype dtype, float softmax_scale, hipStream_t stream) {
  if (!q || !kv_cache || !kv_len || !o) return ATTN_ERR_NULL;
  if (B <= 0 || H <= 0 || d_latent <= 0 || d_rope < 0 || cap <= 0) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_BF16 && dtype != ATTN_F16) {
    if (dtype < ATTN_F32 || dtype > ATTN_FP8_E5M2) return ATTN_ERR_DTYPE;
    return ATTN_ERR_UNSUPPORTED;
  }
  if (d_latent != 448 || d_rope != 64 || H > 16) return ATTN_ERR_UNSUPPORTED;
  split = mla_split(split);
  if (split % 32 != 0 || split < 32 || split > 2048) return ATTN_ERR_SHAPE;
  if (B > 65535) return ATTN_ERR_SHAPE;
  if (!(softmax_scale == softmax_scale)) return ATTN_ERR_SHAPE;
  if (!attn_host::aligned(q, 16) || !attn_host::aligned(kv_cache, 16) ||
      !attn_host::aligned(o, 16) || !attn_host::aligned(kv_len, 4))
    return ATTN_ERR_ALIGN;
  const int nsplit = (cap + split - 1) / split;
  const SplitWorkspace ws = split_workspace((long long)B * H, nsplit, d_latent);
  if (!workspace || workspace_bytes < ws.total) return ATTN_ERR_WORKSPACE;
  if (!attn_host::aligned(workspace, 256)) return ATTN_ERR_ALIGN;

  DecodeMlaParams p{};
  p.q = q; p.c = kv_cache; p.kv_len = kv_len;
  p.o_part = reinterpret_cast<float*>(workspace);
  p.lse_part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + ws.lse_offset);
  p.H = H; p.cap = cap; p.split = split; p.nsplit = nsplit;
  p.scale_log2 = softmax_scale * kLog2e;
  dim3 grid(nsplit, B);
  if (dtype == ATTN_BF16) hipLaunchKernelGGL((decode_mla_split_kernel<Bf16Tag>), grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((decode_mla_split_kernel<F16Tag>), grid, dim3(256), 0, stream, p);
  attn_status st = attn_host::launch_status();
  if (st != ATTN_OK) return st;
  launch_combine(p.o_part, p.lse_part, o, B * H, nsplit, d_latent, dtype, stream);
  return attn_host::launch_status();
}
