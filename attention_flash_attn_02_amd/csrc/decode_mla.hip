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
// One workgroup (4 waves) per (split, sequence); wave w owns dims
// [128 w, 128 w + 128) of every cache row.  The sequence is the fast grid
// dimension, so workgroups are dispatched split by split: every split that
// holds rows comes before the trailing splits of the capacity that lie past
// kv_len (empty, they exit at once).  With the split fastest, those empty
// workgroups were interleaved with the working ones and the dispatcher left
// some compute units with three working workgroups and others with one (B=128,
// capacity 2056: 63.7 us against 56.3 us with capacity 2048).  For each 32-slot
// chunk:
//   * each wave streams its slice of the 32 rows into registers, whole rows
//     per 16-lane group so that every L2 request is a full cache line (the
//     next chunk's loads are in flight while the current one is computed);
//   * the slice rows are staged in the wave's LDS area; each wave computes
//     S^T over its slice from 16-row fragments; the four partial score tiles
//     are summed through LDS (one barrier per chunk), so every wave holds the
//     full scores and runs the identical online softmax;
//   * each wave computes O^T = C_lat^T P^T for the latent dims of its slice,
//     reading the A operand transposed with ds_read_b64_tr_b16.
// Slots at or past kv_len are never loaded; a split that starts past kv_len
// writes the empty partial (o = 0, lse = -inf).  Each split's part is stored
// in bf16 (rounded to nearest even): the part is normalised within its split,
// so the rounding adds at most 2^-9 of its magnitude, on the order of the bf16
// rounding of the output itself, and halves the part traffic (33 MB written
// and read again at batch 128 with fp32 parts, ~10 % of the step's bytes).

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace attn {

struct DecodeMlaParams {
  const void* q;
  const void* c;
  const int32_t* kv_len;
  uint16_t* o_part;  // [B * H, nsplit, d_latent] bf16 bits
  float* lse_part;   // [B * H, nsplit]
  int H, cap, split, nsplit;
  int even;          // 1: part w of a sequence covers the w-th of nsplit equal runs of 32-slot chunks of
                     //    [0, kv_len) (divided on the device); 0: slots [w split, (w + 1) split)
  float scale_log2;
};

typedef __attribute__((ext_vector_type(4))) short v4i16_m;
#define LDS_P(T, ptr) ((__attribute__((address_space(3))) T*)(ptr))

// Chunk buffers per wave: two (one chunk in flight while one is computed)
// keep the kernel at 145 VGPRs, so three workgroups (48 KB of LDS each) share
// a compute unit; with four buffers and two workgroups per compute unit the
// step was 1-10 % slower at every split size.
#ifndef MLA_NBUF
#define MLA_NBUF 2
#endif

template <class Tag, int NBUF = MLA_NBUF>
__global__ __launch_bounds__(256, 3) void decode_mla_split_kernel(const DecodeMlaParams p) {
  constexpr int DQ = 512, DL = 448;
  constexpr int ROWB = 2 * DQ;     // bytes per cache row
  constexpr int SLB = 256;         // bytes of one wave's 128-dim slice of a row
  constexpr int NKK = 4;           // 32-wide k-steps over a slice
  constexpr int NLB = 8;           // 16-row O^T blocks per slice
  __shared__ __attribute__((aligned(1024))) uint8_t cl[4][32 * SLB];  // per-wave slice rows
  __shared__ float sx[2][4][8][64];                                   // partial-score exchange

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int m16 = lane & 15, qq = lane >> 4;
  const int b = blockIdx.x, split_idx = blockIdx.y;
  const int L = min(max(p.kv_len[b], 0), p.cap);
  int s0, s1;
  if (p.even) {  // equal runs of 32-slot chunks, whatever the length
    const int chunks = (L + 31) / 32;
    s0 = 32 * (int)((long long)split_idx * chunks / p.nsplit);
    s1 = min(32 * (int)((long long)(split_idx + 1) * chunks / p.nsplit), L);
  } else {
    s0 = split_idx * p.split;
    s1 = min(s0 + p.split, L);
  }
  const int row0 = b * p.H;
  const int nlb = wave < 3 ? NLB : (DL - 3 * 128) / 16;  // latent blocks in this slice (8, 8, 8, 4)

  if (s0 >= s1) {  // empty split
    for (int idx = tid; idx < p.H * DL; idx += 256)
      p.o_part[((size_t)(row0 + idx / DL) * p.nsplit + split_idx) * DL + idx % DL] = 0;
    if (tid < p.H) p.lse_part[(size_t)(row0 + tid) * p.nsplit + split_idx] = kNegInf;
    return;
  }

  // query fragments of this wave's slice: B operand (column m16 = head)
  u32x4 qf[NKK];
  {
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(p.q) + (size_t)(row0 + m16) * ROWB + SLB * wave;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = m16 < p.H ? ldg16(qrow + 64 * kk + 16 * qq) : u32x4{0, 0, 0, 0};
  }
  // cache rows [s0, s1) of this sequence, this wave's slice, as a raw buffer:
  // a slot at or past s1 lies outside the buffer's range, so its load returns
  // zero without touching memory and every load can be issued unconditionally
  const uint8_t* cbase = reinterpret_cast<const uint8_t*>(p.c) + ((size_t)b * p.cap + s0) * ROWB + SLB * wave;
  const __amdgpu_buffer_rsrc_t crs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(cbase), (short)0, (s1 - s0 - 1) * ROWB + SLB, kBufferRsrcWord3);
  // loads are row-contiguous (a 16-lane group covers one 256-byte slice row),
  // so every L2 request is a full cache line: load j, lane -> row 4 j + lrow,
  // 16-byte chunk lch
  const int lrow = lane >> 4, lch = lane & 15;
  const int lane_off = lrow * ROWB + 16 * lch;
  uint8_t* myl = cl[wave];
  // LDS rows are swizzled by 16-byte chunk: chunk c of row r sits at c ^ swz(r),
  // swz(r) = 2 (r & 7) + ((r >> 3) & 1).  Row-wise stores, 16-row fragment
  // reads (one chunk of 16 rows) and the transposed reads (two adjacent chunks
  // of 4 rows) all hit distinct bank groups.
  auto swz = [](int r) { return ((r & 7) << 1) | ((r >> 3) & 1); };
  const int aswz = swz(m16);
  // transposed reads of the slice rows: group qq reads rows 4 qq + (rr >> 2) (+ 16)
  const int rr = lane & 15;
  const int vrow = 4 * qq + (rr >> 2);
  const int vlane = vrow * SLB + 8 * (rr & 1);
  const int vx = swz(vrow), vq = (rr & 3) >> 1;

  auto load = [&](u32x4 (&cf)[8], int c0) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      cf[j] = __builtin_amdgcn_raw_buffer_load_b128(crs, lane_off + (c0 - s0 + 4 * j) * ROWB, 0, kBufferNontemporal);
    // keep chunks in issue order: each chunk's wait then leaves the later ones in flight
    __builtin_amdgcn_sched_barrier(0);
  };

  f32x4 acc_o[NLB];
#pragma unroll
  for (int i = 0; i < NLB; ++i) acc_o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  int buf = 0;

  auto process = [&](const u32x4 (&cf)[8], int c0) {
    // slice rows -> this wave's LDS area (row-major, swizzled)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 4 * j + lrow;
      *reinterpret_cast<u32x4*>(myl + row * SLB + 16 * (lch ^ swz(row))) = cf[j];
    }
    // partial S^T over this slice (A operand: rows 16 tb + m16, dims 32 kk + 8 qq .. + 7),
    // exchanged and summed over the four slices
    f32x4 sacc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      sacc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(myl + (16 * tb + m16) * SLB + 16 * ((4 * kk + qq) ^ aswz));
        sacc[tb] = Tag::mfma16(a, qf[kk], sacc[tb]);
      }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) sx[buf][wave][r][lane] = sacc[r >> 2][r & 3];
    __syncthreads();
    float sv[8];
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float x = sx[buf][0][r][lane] + sx[buf][1][r][lane] + sx[buf][2][r][lane] + sx[buf][3][r][lane];
      const int tok = c0 + 16 * (r >> 2) + 4 * qq + (r & 3);
      sv[r] = tok < s1 ? x * p.scale_log2 : kNegInf;
      mx = fmaxf(mx, sv[r]);
    }
    buf ^= 1;
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m_run, mx);  // finite: every chunk holds a valid slot
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pv[j] = fast_exp2(sv[j] - m_new);
    const u32x4 pf = {Tag::pack2(pv[0], pv[1]), Tag::pack2(pv[2], pv[3]), Tag::pack2(pv[4], pv[5]),
                      Tag::pack2(pv[6], pv[7])};
    float ps = l_run * alpha;
#pragma unroll
    for (int e = 0; e < 4; ++e) ps = Tag::sum2(pf[e], ps);
    l_run = ps;
    // O^T += C_lat^T P^T over this slice's latent dims
#pragma unroll
    for (int lb = 0; lb < NLB; ++lb) {
      if (lb < nlb) {
        const int off = vlane + 16 * ((2 * lb + vq) ^ vx);
        const v4i16_m x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_P(v4i16_m, myl + off));
        const v4i16_m x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_P(v4i16_m, myl + off + 16 * SLB));
        const u32x2 a1 = __builtin_bit_cast(u32x2, x1), a2 = __builtin_bit_cast(u32x2, x2);
        acc_o[lb] *= alpha;
        acc_o[lb] = Tag::mfma16(u32x4{a1[0], a1[1], a2[0], a2[1]}, pf, acc_o[lb]);
      }
    }
  };

  // NBUF chunk buffers: while one chunk is computed, the next NBUF - 1 are in
  // flight.  Loads are unconditional so the compiler's wait counts stay exact.
  u32x4 cf[NBUF][8];
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i) load(cf[i], s0 + 32 * i);
#pragma unroll 1
  for (int c0 = s0; c0 < s1; c0 += 32 * NBUF) {
#pragma unroll
    for (int i = 0; i < NBUF; ++i) {
      const int c = c0 + 32 * i;
      load(cf[(i + NBUF - 1) % NBUF], c + 32 * (NBUF - 1));
      if (c < s1) process(cf[i], c);
    }
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (m16 < p.H) {
    const float inv = 1.f / l_run;
    const size_t prow = (size_t)(row0 + m16) * p.nsplit + split_idx;
#pragma unroll
    for (int lb = 0; lb < NLB; ++lb)
      if (lb < nlb) {
        const f32x4 v = acc_o[lb] * inv;
        *reinterpret_cast<u32x2*>(p.o_part + prow * DL + 128 * wave + 16 * lb + 4 * qq) =
            u32x2{Bf16Tag::pack2(v[0], v[1]), Bf16Tag::pack2(v[2], v[3])};
      }
    if (wave == 0 && qq == 0) p.lse_part[prow] = (m_run + __log2f(l_run)) * kLn2;
  }
}

}  // namespace attn

using namespace attn;

// Default work division: [0, kv_len) of each sequence is cut on the device
// into n equal runs of 32-slot chunks, one workgroup each, with n chosen
// from the batch so that the launch has about one workgroup per compute
// unit: n = round(CUs / B), at least 1, at most 16 and at most the chunks of
// the capacity.  A workgroup streams its run with two chunks in flight;
// fewer, longer runs at large batch keep the number of parts (and the
// combine's traffic) low, more runs at small batch keep more compute units
// streaming, up to 16 parts, past which merging the parts costs more than
// the shorter runs save (batch 1: 17.5 us with 65 one-chunk parts, 12.8 us
// with 16).  (Fixed splits of 32..2048 slots stay available through `split`.)
static int mla_cu_count() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// parts per sequence (workgroups of one sequence)
static long long mla_parts(int B, int cap, int split) {
  if (split > 0) return (cap + split - 1) / split;
  const long long cus = mla_cu_count();
  const long long n = std::min((cus + B / 2) / B, 16LL);
  return std::max(1LL, std::min(n, (long long)(cap + 31) / 32));
}

extern "C" size_t attn_decode_mla_workspace_bytes(int B, int H, int cap, int d_latent, int split) {
  if (B <= 0 || H <= 0 || cap <= 0 || d_latent <= 0) return 0;
  return split_workspace((long long)B * H, mla_parts(B, cap, split), d_latent, 2).total;
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
  if (split > 0 && (split % 32 != 0 || split < 32 || split > 2048)) return ATTN_ERR_SHAPE;
  if (B > 65535) return ATTN_ERR_SHAPE;
  // the score scale must be a positive finite number, as for the prefill
  if (!(softmax_scale > 0.f) || !(softmax_scale < 3.0e38f)) return ATTN_ERR_SHAPE;
  if (!attn_host::aligned(q, 16) || !attn_host::aligned(kv_cache, 16) ||
      !attn_host::aligned(o, 16) || !attn_host::aligned(kv_len, 4))
    return ATTN_ERR_ALIGN;
  const long long nsplit = mla_parts(B, cap, split);
  if (nsplit > 65535) return ATTN_ERR_SHAPE;
  const SplitWorkspace ws = split_workspace((long long)B * H, nsplit, d_latent, 2);
  if (!workspace || workspace_bytes < ws.total) return ATTN_ERR_WORKSPACE;
  if (!attn_host::aligned(workspace, 256)) return ATTN_ERR_ALIGN;

  DecodeMlaParams p{};
  p.q = q; p.c = kv_cache; p.kv_len = kv_len;
  p.o_part = reinterpret_cast<uint16_t*>(workspace);
  p.lse_part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + ws.lse_offset);
  p.H = H; p.cap = cap; p.split = split; p.nsplit = (int)nsplit; p.even = split <= 0 ? 1 : 0;
  p.scale_log2 = softmax_scale * kLog2e;
  dim3 grid(B, (unsigned)nsplit);
  if (dtype == ATTN_BF16) hipLaunchKernelGGL((decode_mla_split_kernel<Bf16Tag>), grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((decode_mla_split_kernel<F16Tag>), grid, dim3(256), 0, stream, p);
  attn_status st = attn_host::launch_status();
  if (st != ATTN_OK) return st;
  launch_combine_bf16_parts(p.o_part, p.lse_part, o, B * H, (int)nsplit, d_latent, dtype, stream);
  return attn_host::launch_status();
}
