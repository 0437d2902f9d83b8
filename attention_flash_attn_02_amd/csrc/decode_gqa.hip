// Split-context GQA decode ("flash-decoding") against a static KV cache.
//
// Follows the fixed-budget decode audit (sections "Which implementation was
// tested" and "Setup and interpretation"): one new query token per sequence,
// a static append cache (capacity 2056 for a 2048 context), the context cut
// into splits (128 slots in the audit) whose softmax parts are merged, and
// the G query heads of a KV head grouped so one pass over a K/V tile serves
// all of them (the audit notes that such a row tile carries few useful query
// rows; here they ride in the 16-wide N side of a 16x16x32 MFMA).
//
// Here the splits of a KV head are the waves of a workgroup, merged in LDS
// at the end.  When several workgroups share a KV head (the default), each
// writes its part (o, lse) to the workspace and the combine kernel
// (combine.hip) merges them; with one workgroup per KV head the result is
// written directly and a decode step is one kernel.  Slots at or past kv_len are never loaded; a wave or workgroup
// without slots contributes the empty part (o = 0, lse = -inf).

#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace attn {

struct DecodeGqaParams {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* kv_len;
  void* o;          // [B, Hq, D] final output (one workgroup per KV head)
  float* o_part;    // [B * Hq, n_wg, D] partials (several workgroups per KV head)
  float* lse_part;  // [B * Hq, n_wg]
  int Hq, Hkv, G, cap, n_wg, out_dtype;
  float scale_log2;
  int bf16_parts;   // o_part holds bf16 bits instead of fp32
};

typedef __attribute__((ext_vector_type(4))) short v4i16_t;
#define LDS_PTR(T, ptr) ((__attribute__((address_space(3))) T*)(ptr))

// A workgroup of NW waves per (key range, KV head, sequence).  The n_wg
// workgroups of a KV head cut [0, kv_len) into equal runs of 32-slot chunks,
// and the NW waves of a workgroup cut its run the same way, so the work is
// balanced for any length (kv_len is read on the device).  Each wave walks
// its slots in chunks of 32; the next chunk's K and V rows are loaded (into
// a second register set) while the current chunk is computed, so loads stay
// in flight the whole time.  Rows are loaded whole so that every L2 request
// is a full cache line, and staged in the wave's LDS area:
//   * K fragments (16 rows x 32 dims) are read back as the A operand of
//     S^T = K Q^T;
//   * V rows are read back transposed with ds_read_b64_tr_b16, which yields
//     the A operand of O^T = V^T P^T directly.
// The waves' softmax parts are then merged through LDS (the merge of
// softmax parts of the fixed-budget decode audit, section "A: group-entry
// queries and one joint history scan", as one weighted sum): with a single
// workgroup per KV head the result is final and is written in the output
// type; otherwise the workgroup's part (normalised o, lse) goes to the
// workspace and the combine kernel merges the parts.
template <class Tag, int NW>
__global__ __launch_bounds__(64 * NW, 2) void decode_gqa_kernel(const DecodeGqaParams p) {
  constexpr int D = 128;
  constexpr int ROWB = 2 * D;  // bytes per cache row
  constexpr int NDB = D / 16;  // 16-row blocks of O^T
  constexpr int NKK = D / 32;  // 32-wide k-steps of S^T
  constexpr int NBUF = 2;
  // per wave: V rows and K rows of the chunk (reused for the merge)
  __shared__ __attribute__((aligned(1024))) uint8_t stage[NW][2][32 * ROWB];

  // the wave index in a scalar register: the wave's slot range, and with it
  // the K/V buffer descriptors, are then wave-uniform, and the buffer loads
  // take them as they are instead of looping over distinct per-lane values
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint8_t* vs = stage[wave][0];
  uint8_t* ks = stage[wave][1];
  const int m16 = lane & 15, qq = lane >> 4;
  const int wg = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int row0 = b * p.Hq + kvh * p.G;  // first query head (output row) of this KV head
  // query fragments (B operand of S^T; columns m16 < G are real heads),
  // loaded before the cache length is read so that the two loads overlap
  constexpr int NKKQ = D / 32;
  u32x4 qf[NKKQ];
  {
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(p.q) + (size_t)(row0 + min(m16, p.G - 1)) * ROWB;
#pragma unroll
    for (int kk = 0; kk < NKKQ; ++kk) qf[kk] = ldg16(qrow + 64 * kk + 16 * qq);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int L = min(max(p.kv_len[b], 0), p.cap);
  // chunk range of this workgroup, then of this wave
  const int nch = (L + 31) >> 5;
  const int cpg = (nch + p.n_wg - 1) / p.n_wg;
  const int gc0 = min(wg * cpg, nch), gc1 = min(gc0 + cpg, nch);
  const int cpw = (gc1 - gc0 + NW - 1) / NW;
  const int wc0 = min(gc0 + wave * cpw, gc1), wc1 = min(wc0 + cpw, gc1);
  const int s0 = wc0 * 32;
  const int s1 = min(wc1 * 32, L);

  f32x4 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  if (s0 < s1) {
    // columns m16 >= G are not heads: zero them (loaded from head G - 1)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      if (m16 >= p.G) qf[kk] = u32x4{0, 0, 0, 0};

    // K and V rows [s0, s1) of this (sequence, KV head) as raw buffers: a slot
    // at or past s1 lies outside the buffer's range, so its load returns zero
    // without touching memory and every load can be issued unconditionally
    const size_t kv_base = ((size_t)b * p.Hkv + kvh) * p.cap + s0;
    const int range = (s1 - s0) * ROWB;
    const __amdgpu_buffer_rsrc_t krs_s = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(p.kc) + kv_base * ROWB), (short)0, range, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs_s = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(p.vc) + kv_base * ROWB), (short)0, range, kBufferRsrcWord3);
    // V staging: lane holds chunk vdc of rows 8 vtg .. 8 vtg + 7
    const int vdc = lane & 15, vtg = lane >> 4;
    // transposed V reads: group qq reads rows 4 qq + (rr >> 2) (+ 16), dims 16 db + 4 (rr & 3)
    const int rr = lane & 15;
    int voff[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int row = 4 * qq + (rr >> 2), d = 16 * db + 4 * (rr & 3);
      voff[db] = row * ROWB + 16 * ((d >> 3) ^ (2 * (row & 7))) + 2 * (d & 7);
    }

    // K and V rows are loaded whole (a 16-lane group covers one 256-byte row),
    // so every request to L2 is a full cache line:
    //   K: load j, lane -> row 4 j + (lane >> 4), 16-byte chunk lane & 15
    //   V: load r, lane -> row 8 vtg + r, chunk vdc
    const int krow = lane >> 4, kch = lane & 15;
    auto load = [&](u32x4 (&kr)[8], u32x4 (&vr)[8], int c0) {
      const int cb = (c0 - s0) * ROWB;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        kr[j] = __builtin_amdgcn_raw_buffer_load_b128(krs_s, cb + (4 * j + krow) * ROWB + 16 * kch, 0, kBufferNontemporal);
#pragma unroll
      for (int r = 0; r < 8; ++r)
        vr[r] = __builtin_amdgcn_raw_buffer_load_b128(vrs_s, cb + (8 * vtg + r) * ROWB + 16 * vdc, 0, kBufferNontemporal);
      // keep chunks in issue order: each chunk's wait then leaves the later ones in flight
      __builtin_amdgcn_sched_barrier(0);
    };

    auto process = [&](const u32x4 (&kr)[8], const u32x4 (&vr)[8], int c0) {
      // K and V rows of the chunk -> LDS (row-major).  K chunk swizzle row & 15
      // keeps both the row-wise stores and the 16-row fragment reads below
      // conflict-free; V keeps 2 (row & 7) for the transposed reads.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = 4 * j + krow;
        *reinterpret_cast<u32x4*>(ks + row * ROWB + 16 * (kch ^ (row & 15))) = kr[j];
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int row = 8 * vtg + r;
        *reinterpret_cast<u32x4*>(vs + row * ROWB + 16 * (vdc ^ (2 * (row & 7)))) = vr[r];
      }
      // S^T = K Q^T: A operand = K rows 16 tb + m16, dims 32 kk + 8 qq .. + 7;
      // lane holds slots 16 tb + 4 qq + i of query column m16
      f32x4 sacc[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        sacc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(ks + (16 * tb + m16) * ROWB + 16 * ((4 * kk + qq) ^ m16));
          sacc[tb] = Tag::mfma16(a, qf[kk], sacc[tb]);
        }
      }
      float sv[8];
      float mx = kNegInf;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = c0 + 16 * tb + 4 * qq + i;
          const float x = tok < s1 ? sacc[tb][i] * p.scale_log2 : kNegInf;
          sv[4 * tb + i] = x;
          mx = fmaxf(mx, x);
        }
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
      // O^T += V^T P^T; slot j of quarter qq is chunk row 16 (j / 4) + 4 qq + j % 4
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const v4i16_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16_t, vs + voff[db]));
        const v4i16_t x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16_t, vs + voff[db] + 16 * ROWB));
        const u32x2 a1 = __builtin_bit_cast(u32x2, x1), a2 = __builtin_bit_cast(u32x2, x2);
        acc_o[db] *= alpha;
        acc_o[db] = Tag::mfma16(u32x4{a1[0], a1[1], a2[0], a2[1]}, pf, acc_o[db]);
      }
    };

    // NBUF chunk buffers: while one chunk is computed, the next NBUF - 1 are in
    // flight.  Loads are unconditional so the compiler's wait counts stay exact.
    u32x4 kr[NBUF][8], vr[NBUF][8];
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) load(kr[i], vr[i], s0 + 32 * i);
#pragma unroll 1
    for (int c0 = s0; c0 < s1; c0 += 32 * NBUF) {
#pragma unroll
      for (int i = 0; i < NBUF; ++i) {
        const int c = c0 + 32 * i;
        load(kr[(i + NBUF - 1) % NBUF], vr[(i + NBUF - 1) % NBUF], c + 32 * (NBUF - 1));
        if (c < s1) process(kr[i], vr[i], c);
      }
    }
  }
  // row sum of this wave's part: lanes (m16, qq) over qq
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // ---- merge the NW waves' parts through LDS ----
  // wave w's area (its own staging, free once its loop is done):
  //   o: [NDB][64 lanes] float4 = O^T[16 db + 4 qq + i][m16] (unnormalised);
  //   m, l of each query column after it
  auto area = [&](int w) { return reinterpret_cast<float*>(&stage[w][0][0]); };  // 16 KB per wave
  float* mo = area(wave);
  float* ml = mo + NDB * 64 * 4;
#pragma unroll
  for (int db = 0; db < NDB; ++db) *reinterpret_cast<f32x4*>(mo + (db * 64 + lane) * 4) = acc_o[db];
  if (qq == 0) {
    ml[m16] = m_run;
    ml[16 + m16] = l_run;
  }
  __syncthreads();
  // wave w finishes O^T blocks db = w, w + NW, ... for every query column
  float mw[NW], M = kNegInf;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mw[w] = area(w)[NDB * 64 * 4 + m16];
    M = fmaxf(M, mw[w]);
  }
  float fw[NW], Lsum = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    fw[w] = M == kNegInf ? 0.f : fast_exp2(mw[w] - M);  // 0 for a wave without slots
    Lsum += fw[w] * area(w)[NDB * 64 * 4 + 16 + m16];
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  const bool direct = p.n_wg == 1;
  if (m16 < p.G) {
    const size_t row = (size_t)(row0 + m16);
    const size_t prow = row * p.n_wg + wg;
#pragma unroll
    for (int db = wave; db < NDB; db += NW) {
      f32x4 o4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w)
        o4 += fw[w] * *reinterpret_cast<const f32x4*>(area(w) + (db * 64 + lane) * 4);
      o4 *= inv;
      if (direct) store4(p.o, row * D + 16 * db + 4 * qq, p.out_dtype, o4[0], o4[1], o4[2], o4[3]);
      else if (p.bf16_parts)
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.o_part) + prow * D + 16 * db + 4 * qq) =
            u32x2{Bf16Tag::pack2(o4[0], o4[1]), Bf16Tag::pack2(o4[2], o4[3])};
      else *reinterpret_cast<f32x4*>(p.o_part + prow * D + 16 * db + 4 * qq) = o4;
    }
    if (!direct && wave == 0 && qq == 0)
      p.lse_part[prow] = Lsum > 0.f ? (M + __log2f(Lsum)) * kLn2 : kNegInf;
  }
}

// waves per workgroup
constexpr int kGqaWaves = 4;

template <class Tag>
static void launch_decode(const DecodeGqaParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_gqa_kernel<Tag, kGqaWaves>), grid, dim3(64 * kGqaWaves), 0, st, p);
}

}  // namespace attn

using namespace attn;

// split: the most slots one wave streams.  A KV head gets
// n_wg = ceil(cap / (waves * split)) workgroups.  The default, 128 (the
// decode audit's split size), gives five workgroups per KV head at capacity
// 2056: enough workgroups to fill the chip from batch 1, and a combine step
// over five parts.  Splits of 1024 give one workgroup per KV head up to
// capacity 4096 and no combine step (fastest only at large batch).
static const int kDefaultGqaSplit = 128;

static int gqa_split(int split) { return split <= 0 ? kDefaultGqaSplit : split; }

static int gqa_n_wg(int cap, int split) {
  const long long per_wg = (long long)kGqaWaves * split;
  return (int)((cap + per_wg - 1) / per_wg);
}

extern "C" size_t attn_decode_gqa_workspace_bytes(int B, int Hq, int cap, int D, int split) {
  split = gqa_split(split);
  if (B <= 0 || Hq <= 0 || cap <= 0 || D <= 0 || split <= 0) return 0;
  const int n_wg = gqa_n_wg(cap, split);
  if (n_wg <= 1) return 0;
  return split_workspace((long long)B * Hq, n_wg, D).total;
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
  // the score scale must be a positive finite number, as for the prefill
  if (!(softmax_scale > 0.f) || !(softmax_scale < 3.0e38f)) return ATTN_ERR_SHAPE;
  if (!attn_host::aligned(q, 16) || !attn_host::aligned(k_cache, 16) ||
      !attn_host::aligned(v_cache, 16) || !attn_host::aligned(o, 16) ||
      !attn_host::aligned(kv_len, 4))
    return ATTN_ERR_ALIGN;
  const int n_wg = gqa_n_wg(cap, split);

  DecodeGqaParams p{};
  p.q = q; p.kc = k_cache; p.vc = v_cache; p.kv_len = kv_len; p.o = o;
  p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.cap = cap; p.n_wg = n_wg; p.out_dtype = dtype;
  p.scale_log2 = softmax_scale * kLog2e;
  // parts as bf16 from 1024 query rows on: half the part bytes, which the
  // large batches feel (B = 128: 88.0 -> 84.8 us); below that the fp32 parts'
  // combine, which loads every part up front, is the quicker one (B = 1 and 8:
  // 0.3 us)
  p.bf16_parts = (long long)B * Hq >= 1024;
  if (n_wg > 1) {
    const SplitWorkspace ws = split_workspace((long long)B * Hq, n_wg, D);
    if (!workspace || workspace_bytes < ws.total) return ATTN_ERR_WORKSPACE;
    if (!attn_host::aligned(workspace, 256)) return ATTN_ERR_ALIGN;
    p.o_part = reinterpret_cast<float*>(workspace);
    p.lse_part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + ws.lse_offset);
  }
  const dim3 grid(n_wg, Hkv, B);
  if (dtype == ATTN_BF16) launch_decode<Bf16Tag>(p, grid, stream);
  else launch_decode<F16Tag>(p, grid, stream);
  attn_status st = attn_host::launch_status();
  if (st != ATTN_OK || n_wg == 1) return st;
  if (p.bf16_parts)
    launch_combine_bf16_parts(reinterpret_cast<const uint16_t*>(p.o_part), p.lse_part, o, B * Hq, n_wg, D, dtype,
                              stream);
  else
    launch_combine(p.o_part, p.lse_part, o, B * Hq, n_wg, D, dtype, stream);
  return attn_host::launch_status();
}

// ---------------------------------------------------------------------------
// Allocation-free form: the split partials go to a file-scope device array
// instead of a caller workspace.  The array's name is only a host-side
// stand-in for the symbol; its device address (one per GPU) comes from
// hipGetSymbolAddress on the first call on that GPU, and only that address
// is passed to the kernels.  Every call on a GPU shares its array, so calls
// that overlap on one GPU (two streams, two threads) race.  Nothing in it
// needs clearing: the split kernel writes every part slot (empty ranges as
// o = 0, lse = -inf) before the combine kernel reads it.
// ---------------------------------------------------------------------------
static constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;  // 8 MiB per GPU
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static constexpr int kMaxDevices = 64;

// device address of this GPU's scratch (the current device), or null
static void* scratch_address() {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

extern "C" attn_status attn_decode_gqa_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                               const int32_t* kv_len, void* o, int B, int Hq, int Hkv, int D,
                                               int cap, int split, attn_dtype dtype, float softmax_scale,
                                               hipStream_t stream) {
  const size_t need = attn_decode_gqa_workspace_bytes(B, Hq, cap, D, split);
  if (need > kNoAllocScratchBytes) return ATTN_ERR_WORKSPACE;  // beyond the static scratch
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_address();
    if (!ws) return ATTN_ERR_LAUNCH;
  }
  return attn_decode_gqa(q, k_cache, v_cache, kv_len, o, ws, need, B, Hq, Hkv, D, cap, split, dtype,
                         softmax_scale, stream);
}
