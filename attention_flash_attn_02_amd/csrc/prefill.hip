// Prefill attention forward with online softmax (causal or not, GQA, fused
// RoPE) for gfx950.
//
// Operation (textbook scaled-dot-product attention, which the pages name but
// do not print): for query head h, KV head g = h / G,
//   O[i] = sum_j softmax_j(scale * <rope(q_i, i), rope(k_j, j)>) v_j
// over j <= i when causal.  RoPE fused into the attention kernel follows the
// shape-adaptive attention lesson page (rows "What was tried" and
// "Conditions": causal GQA prefill with RoPE-attention fusion); fp8 e5m2
// inputs follow the persistent-attention digest (benchmark section).
//
// MFMA kernel (f16, bf16, fp8 e5m2 inputs; D = 64 or 128):
//   * A workgroup is 4 waves; each wave owns 32 query rows of one head.  For
//     GQA the 4 waves take consecutive heads of one KV group at the same
//     positions, so one K/V tile staged in LDS serves all of them and the
//     causal bound is the same for the whole workgroup.
//   * Scores are computed transposed, S^T = K Q^T, on 32x32 MFMA tiles: K
//     comes from LDS as the A operand and Q stays in registers as the B
//     operand.  Each lane then holds one query row, so the row max and row
//     sum need a single cross-lane step (lane l and l^32).
//   * The probabilities leave the accumulator already in B-operand layout for
//     O^T = V^T P^T; V is staged transposed in LDS (keys contiguous, with the
//     key order inside each 16-key block permuted to match the accumulator)
//     so that the A operand is one 16-byte LDS read.
//   * RoPE on K is applied while staging each K tile, with the angle split
//     into a per-tile base (table in LDS) and a per-row offset (registers):
//     cos/sin of (t0 + r) w from cos/sin(t0 w) and cos/sin(r w).
//   * Work items are issued longest-first (causal tiles near the end of the
//     sequence first) so short tiles fill the tail of the launch.
// fp32 inputs use a plain SIMT kernel (one query row per thread).

#include "common.hpp"

namespace attn {

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, S;
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
  double rope_frev[64];  // the same frequencies in revolutions per position (/ 2 pi)
};

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------
template <class Tag, int D, bool CAUSAL, bool ROPE, bool FP8>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(const PrefillParams p) {
  constexpr int BN = 64;                 // keys per tile
  constexpr int KB = FP8 ? 1 : 2;        // bytes per K element in LDS
  constexpr int KPITCH = D * KB + 16;    // bytes per K row in LDS (padded)
  constexpr int VPITCH = BN + 8;         // 16-bit elements per V^T row in LDS
  constexpr int NKK = D / 16;            // 16-wide k-steps over D (16-bit types)
  constexpr int NDB = D / 32;            // 32-row blocks of O^T
  constexpr int HALF = D / 2;
  constexpr int KPT = D / 32;            // V keys per thread when staging
  constexpr int NKG = BN / KPT;          // V key groups
  constexpr int PAIRS = D / 64;          // K chunk pairs per thread when staging
  constexpr int QREGS = FP8 ? D / 8 : D / 4;   // dwords of Q fragments per lane

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[BN * KPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * VPITCH];
  __shared__ float rope_base[2][D];  // [cos(D/2) | sin(D/2)] of the tile's first position

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int m = lane & 31;   // query row of this lane inside the wave
  const int hh = lane >> 5;  // k half

  // ---- work item: longest (last positions) first ----
  const int per_ptile = p.B * p.Hkv * p.n_hgroups;
  const int item = blockIdx.x;
  const int ptile = p.n_ptiles - 1 - item / per_ptile;
  int rest = item % per_ptile;
  const int hg = rest % p.n_hgroups;
  rest /= p.n_hgroups;
  const int kvh = rest % p.Hkv;
  const int b = rest / p.Hkv;
  const int head = kvh * p.G + hg * p.GP + (wave % p.GP);
  const int p0 = ptile * p.P;
  const int pw0 = p0 + (wave / p.GP) * 32;
  const int kend = CAUSAL ? min(p.S, p0 + p.P) : p.S;
  const int n_kt = (kend + BN - 1) / BN;
  const int qpos = pw0 + m;

  // ---- Q fragments (B operand of S^T = K Q^T), rotated and kept in registers ----
  uint32_t qf[QREGS];
  {
    const size_t qoff = (((size_t)b * p.Hq + head) * p.S + qpos) * D;
    if (FP8) {
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(p.q) + qoff;
#pragma unroll
      for (int u = 0; u < D / 64; ++u) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          u32x4 w = qpos < p.S ? ldg16(qrow + 64 * u + 32 * hh + 16 * c) : u32x4{0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 4; ++e) qf[8 * u + 4 * c + e] = w[e];
        }
      }
    } else {
      const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + qoff;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        u32x4 w = qpos < p.S ? ldg16(qrow + 16 * kk + 8 * hh) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[4 * kk + e] = w[e];
      }
      if (ROPE) {
        // element j of k-step kk sits at d = 16 kk + 8 hh + j; its rotate-half
        // partner d + D/2 is in k-step kk + D/32 of the same lane.
#pragma unroll
        for (int kk = 0; kk < NKK / 2; ++kk) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w1 = qf[4 * kk + e], w2 = qf[4 * (kk + NKK / 2) + e];
            float r1[2], r2[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const int i = 16 * kk + 8 * hh + 2 * e + s;
              float sn, cs;
              sincosf((float)qpos * p.inv_freq[i], &sn, &cs);
              const float x1 = Tag::to_f32(s ? (w1 >> 16) : (w1 & 0xffff));
              const float x2 = Tag::to_f32(s ? (w2 >> 16) : (w2 & 0xffff));
              r1[s] = x1 * cs - x2 * sn;
              r2[s] = x2 * cs + x1 * sn;
            }
            qf[4 * kk + e] = Tag::pack2(r1[0], r1[1]);
            qf[4 * (kk + NKK / 2) + e] = Tag::pack2(r2[0], r2[1]);
          }
        }
      }
    }
  }

  // ---- staging assignment ----
  // K: row kr of the tile, chunk pairs (kj + 4u, kj + 4u + D/16) of 8 elements
  const int kr = tid >> 2, kj = tid & 3;
  // V: keys vn0 .. vn0 + KPT - 1, d = 8 * vdc .. 8 * vdc + 7
  const int vdc = tid / NKG, vkg = tid % NKG, vn0 = vkg * KPT;
  // position of key n inside its 16-key block of V^T: groups of 4 keys in
  // order 0, 2, 1, 3 (matches the accumulator's key order)
  const int vg = (vn0 & 15) >> 2;
  const int vpos = (vn0 & ~15) + 4 * (vg == 1 ? 2 : vg == 2 ? 1 : vg) + (vn0 & 3);

  const size_t kv_base = ((size_t)b * p.Hkv + kvh) * p.S;
  const uint8_t* kptr = reinterpret_cast<const uint8_t*>(p.k);
  const uint8_t* vptr = reinterpret_cast<const uint8_t*>(p.v);

  // register staging buffers for the next tile
  u32x4 kbuf[FP8 ? 1 : 2 * PAIRS];
  u32x2 kbuf8[FP8 ? 2 * PAIRS : 1];
  u32x4 vbuf[FP8 ? 1 : KPT];
  u32x2 vbuf8[FP8 ? KPT : 1];
  (void)kbuf8; (void)vbuf8; (void)kbuf; (void)vbuf;

  // per-thread RoPE row offsets cos/sin(kr * w_i) for the thread's frequencies
  float rc[ROPE ? 8 * PAIRS : 1], rs[ROPE ? 8 * PAIRS : 1];
  if (ROPE) {
#pragma unroll
    for (int u = 0; u < PAIRS; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) sincosf((float)kr * p.inv_freq[8 * (kj + 4 * u) + j], &rs[8 * u + j], &rc[8 * u + j]);
  }

  auto load_tile = [&](int t) {
    const int key = t * BN + kr;
    if (FP8) {
      // D bytes per row; thread covers D/4 bytes as 8-byte pieces
#pragma unroll
      for (int u = 0; u < 2 * PAIRS; ++u)
        kbuf8[u] = key < p.S ? ldg8(kptr + (kv_base + key) * D + (D / 4) * kj + 8 * u) : u32x2{0, 0};
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const int vk = t * BN + vn0 + r;
        vbuf8[r] = vk < p.S ? ldg8(vptr + (kv_base + vk) * D + 8 * vdc) : u32x2{0, 0};
      }
    } else {
#pragma unroll
      for (int u = 0; u < PAIRS; ++u) {
        const int c = kj + 4 * u;
        kbuf[2 * u] = key < p.S ? ldg16(kptr + ((kv_base + key) * D + 8 * c) * 2) : u32x4{0, 0, 0, 0};
        kbuf[2 * u + 1] = key < p.S ? ldg16(kptr + ((kv_base + key) * D + 8 * c + HALF) * 2) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const int vk = t * BN + vn0 + r;
        vbuf[r] = vk < p.S ? ldg16(vptr + ((kv_base + vk) * D + 8 * vdc) * 2) : u32x4{0, 0, 0, 0};
      }
    }
  };

  auto rope_base_fill = [&](int t, int slot) {
    if (ROPE && tid < HALF) {
      float sn, cs;
      sincosf((float)(t * BN) * p.inv_freq[tid], &sn, &cs);
      rope_base[slot][tid] = cs;
      rope_base[slot][HALF + tid] = sn;
    }
  };

  auto stage_tile = [&](int t) {
    // ---- K (rotated) -> LDS ----
    if (FP8) {
#pragma unroll
      for (int u = 0; u < 2 * PAIRS; ++u)
        *reinterpret_cast<u32x2*>(k_lds + kr * KPITCH + (D / 4) * kj + 8 * u) = kbuf8[u];
    } else {
#pragma unroll
      for (int u = 0; u < PAIRS; ++u) {
        const int c = kj + 4 * u;
        u32x4 lo = kbuf[2 * u], hi = kbuf[2 * u + 1];
        if (ROPE) {
          const int slot = t & 1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float r1[2], r2[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const int j = 2 * e + s;
              const int i = 8 * c + j;
              const float cb = rope_base[slot][i], sb = rope_base[slot][HALF + i];
              const float cs = cb * rc[8 * u + j] - sb * rs[8 * u + j];
              const float sn = sb * rc[8 * u + j] + cb * rs[8 * u + j];
              const float x1 = Tag::to_f32(s ? (lo[e] >> 16) : (lo[e] & 0xffff));
              const float x2 = Tag::to_f32(s ? (hi[e] >> 16) : (hi[e] & 0xffff));
              r1[s] = x1 * cs - x2 * sn;
              r2[s] = x2 * cs + x1 * sn;
            }
            lo[e] = Tag::pack2(r1[0], r1[1]);
            hi[e] = Tag::pack2(r2[0], r2[1]);
          }
        }
        *reinterpret_cast<u32x4*>(k_lds + kr * KPITCH + 16 * c) = lo;
        *reinterpret_cast<u32x4*>(k_lds + kr * KPITCH + 16 * c + HALF * 2) = hi;
      }
    }
    // ---- V -> LDS, transposed: v_lds[d][pos] ----
    uint32_t w[KPT][4];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      if (FP8) {
        w[r][0] = e5m2x2_to_f16x2(vbuf8[r][0] & 0xffff);
        w[r][1] = e5m2x2_to_f16x2(vbuf8[r][0] >> 16);
        w[r][2] = e5m2x2_to_f16x2(vbuf8[r][1] & 0xffff);
        w[r][3] = e5m2x2_to_f16x2(vbuf8[r][1] >> 16);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) w[r][e] = vbuf[r][e];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t* dst = v_lds + (8 * vdc + i) * VPITCH + vpos;
      const int e = i >> 1;
      if (KPT == 4) {
        u32x2 o;
        o[0] = (i & 1) ? ((w[0][e] >> 16) | (w[1][e] & 0xffff0000u)) : ((w[0][e] & 0xffffu) | (w[1][e] << 16));
        o[1] = (i & 1) ? ((w[2][e] >> 16) | (w[3][e] & 0xffff0000u)) : ((w[2][e] & 0xffffu) | (w[3][e] << 16));
        *reinterpret_cast<u32x2*>(dst) = o;
      } else {
        const uint32_t o = (i & 1) ? ((w[0][e] >> 16) | (w[1][e] & 0xffff0000u)) : ((w[0][e] & 0xffffu) | (w[1][e] << 16));
        *reinterpret_cast<uint32_t*>(dst) = o;
      }
    }
  };

  // ---- running state ----
  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_run = kNegInf;  // running max (scaled log2 domain)
  float l_run = 0.f;      // running sum over this lane's keys

  rope_base_fill(0, 0);
  load_tile(0);

  for (int t = 0; t < n_kt; ++t) {
    __syncthreads();  // previous tile's LDS reads are done; rope base of tile t visible
    stage_tile(t);
    if (t + 1 < n_kt) {
      rope_base_fill(t + 1, (t + 1) & 1);
      load_tile(t + 1);
    }
    __syncthreads();

    const int key0 = t * BN;
    // whole tile invisible to this wave (all keys after all its rows)?
    if (CAUSAL && key0 > pw0 + 31) continue;

    // ---- S^T = K Q^T ----
    f32x16 acc_s[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      acc_s[nb] = f32x16{};
      const uint8_t* krow = k_lds + (32 * nb + m) * KPITCH;
      if (FP8) {
#pragma unroll
        for (int u = 0; u < D / 64; ++u) {
          u32x4 a0 = *reinterpret_cast<const u32x4*>(krow + 64 * u + 32 * hh);
          u32x4 a1 = *reinterpret_cast<const u32x4*>(krow + 64 * u + 32 * hh + 16);
          i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          i32x8 bq;
#pragma unroll
          for (int e = 0; e < 8; ++e) bq[e] = (int)qf[8 * u + e];
          acc_s[nb] = mfma32_bf8(a, bq, acc_s[nb]);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          u32x4 a = *reinterpret_cast<const u32x4*>(krow + 32 * kk + 16 * hh);
          u32x4 bq = {qf[4 * kk], qf[4 * kk + 1], qf[4 * kk + 2], qf[4 * kk + 3]};
          acc_s[nb] = Tag::mfma32(a, bq, acc_s[nb]);
        }
      }
    }

    // ---- mask + online softmax (this lane: query row qpos, 32 keys) ----
    const bool need_mask = (key0 + BN > p.S) || (CAUSAL && key0 + BN - 1 > pw0);
    float mx = kNegInf;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = acc_s[nb][i] * p.scale_log2;
        if (need_mask) {
          const int key = key0 + 32 * nb + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (key >= p.S || (CAUSAL && key > qpos)) s = kNegInf;
        }
        acc_s[nb][i] = s;
        mx = fmaxf(mx, s);
      }
    }
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
    uint32_t pf[4][4];  // P fragments for the 4 16-key steps
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float e0 = fast_exp2(acc_s[nb][i] - m_use);
        const float e1 = fast_exp2(acc_s[nb][i + 1] - m_use);
        psum += e0 + e1;
        const int c = 2 * nb + (i >> 3);
        pf[c][(i & 7) >> 1] = (FP8 ? F16Tag::pack2(e0, e1) : Tag::pack2(e0, e1));
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint16_t* vrow = v_lds + (32 * db + m) * VPITCH;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u32x4 a = *reinterpret_cast<const u32x4*>(vrow + 16 * c + 8 * hh);
        u32x4 bp = {pf[c][0], pf[c][1], pf[c][2], pf[c][3]};
        if (FP8) acc_o[db] = F16Tag::mfma32(a, bp, acc_o[db]);
        else acc_o[db] = Tag::mfma32(a, bp, acc_o[db]);
      }
    }
  }

  // ---- epilogue ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? p.out_scale / l_tot : 0.f;
  if (qpos < p.S) {
    const size_t obase = (((size_t)b * p.Hq + head) * p.S + qpos) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hh;
        store4(p.o, obase + d, p.out_dtype, acc_o[db][4 * g] * inv, acc_o[db][4 * g + 1] * inv,
               acc_o[db][4 * g + 2] * inv, acc_o[db][4 * g + 3] * inv);
      }
    if (p.lse && hh == 0) {
      p.lse[((size_t)b * p.Hq + head) * p.S + qpos] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA kernel, 16-bit inputs: 8 waves per workgroup.
//
// The two halves of the workgroup (waves 0-3 and 4-7) hold the same 128 query
// rows and split the key tiles of the item between them (even / odd tiles);
// their softmax partials are merged through LDS at the end of the item.  For
// causal attention each workgroup takes a long item and the matching short
// one (items k and n-1-k of the longest-first order), so every workgroup has
// the same amount of work.
//
// K and V tiles go straight from HBM to LDS (global_load_lds, 16 B per lane)
// into XOR-swizzled row-major layouts, double buffered, with one barrier per
// key tile.  V is read transposed by ds_read_b64_tr_b16: each 16-lane group
// reads a 4-key x 16-dim block and every lane receives one dim column of 4
// keys, which is exactly the A operand of O^T = V^T P^T.  With RoPE the K
// tile is instead loaded into registers, rotated and written to LDS.
// The running row maximum is only moved when a row's new maximum exceeds it
// by more than 2^8 (lazy rescaling; the result is exact, the probabilities
// just stay below 256 in the meantime).
// ---------------------------------------------------------------------------
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

template <class Tag, int D, bool CAUSAL, bool ROPE>
__global__ __launch_bounds__(512) void prefill_v2_kernel(const PrefillParams p) {
  constexpr int BN = 64;
  constexpr int ROWB = D * 2;        // bytes per K/V row
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int TILEB = BN * ROWB;   // bytes of one K or V tile
  constexpr int RPI = 64 / CH;       // rows per wave-wide direct load
  constexpr int IPW = BN / RPI / 4;  // direct loads per wave per tile
  constexpr int NKK = D / 16, NDB = D / 32, HALF = D / 2, PAIRS = D / 64;
  constexpr float kLazy = 8.f;       // rescale only when the max grows by > 2^8

  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * 2 * 2 * TILEB];  // [half][stage][K,V]
  __shared__ float rope_base[2][2][ROPE ? D : 1];  // [half][slot][rev0 | freq]: see rope_base_fill

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = wave >> 2, wq = wave & 3, htid = tid & 255;
  const int m = lane & 31, hh = lane >> 5;
  uint8_t* hbuf = smem + half * (4 * TILEB);

  const int per_ptile = p.B * p.Hkv * p.n_hgroups;
  const int n_items = p.n_ptiles * per_ptile;
  const int item_long = blockIdx.x;
  const int item_short = n_items - 1 - (int)blockIdx.x;
  const int n_my = (CAUSAL && item_short > item_long) ? 2 : 1;

  // RoPE staging of K: row kr, chunk pairs (kj + 4u, kj + 4u + CH/2)
  const int kr = htid >> 2, kj = htid & 3;

#pragma unroll 1
  for (int itn = 0; itn < n_my; ++itn) {
    if (itn > 0) __syncthreads();  // LDS of the previous item is free
    const int item = itn == 0 ? item_long : item_short;
    const int ptile = p.n_ptiles - 1 - item / per_ptile;
    int rest = item % per_ptile;
    const int hg = rest % p.n_hgroups;
    rest /= p.n_hgroups;
    const int kvh = rest % p.Hkv;
    const int b = rest / p.Hkv;
    const int head = kvh * p.G + hg * p.GP + (wq % p.GP);
    const int p0 = ptile * p.P;
    const int pw0 = p0 + (wq / p.GP) * 32;
    const int kend = CAUSAL ? min(p.S, p0 + p.P) : p.S;
    const int n_kt = (kend + BN - 1) / BN;
    const int n_it = (n_kt + 1) >> 1;  // iterations; this half takes tile 2 i + half
    const int qpos = pw0 + m;

    // ---- Q fragments (B operand of S^T = K Q^T) ----
    uint32_t qf[D / 4];
    {
      const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + (((size_t)b * p.Hq + head) * p.S + qpos) * D;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        u32x4 w = qpos < p.S ? ldg16(qrow + 16 * kk + 8 * hh) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[4 * kk + e] = w[e];
      }
      if (ROPE) {
#pragma unroll
        for (int kk = 0; kk < NKK / 2; ++kk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w1 = qf[4 * kk + e], w2 = qf[4 * (kk + NKK / 2) + e];
            float r1[2], r2[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              // angle in revolutions, reduced exactly in fp64; v_sin/v_cos take revolutions
              const double rv = (double)qpos * p.rope_frev[16 * kk + 8 * hh + 2 * e + s];
              const float rev = (float)(rv - floor(rv));
              const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
              const float x1 = Tag::to_f32(s ? (w1 >> 16) : (w1 & 0xffff));
              const float x2 = Tag::to_f32(s ? (w2 >> 16) : (w2 & 0xffff));
              r1[s] = x1 * cs - x2 * sn;
              r2[s] = x2 * cs + x1 * sn;
            }
            qf[4 * kk + e] = Tag::pack2(r1[0], r1[1]);
            qf[4 * (kk + NKK / 2) + e] = Tag::pack2(r2[0], r2[1]);
          }
      }
    }

    const size_t kv_row0 = ((size_t)b * p.Hkv + kvh) * p.S;
    const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.k) + kv_row0 * ROWB;
    const uint8_t* vg = reinterpret_cast<const uint8_t*>(p.v) + kv_row0 * ROWB;

    // direct HBM -> LDS load of one K or V tile (rows past S re-read row S-1;
    // those keys are masked and their probabilities are exactly zero)
    auto dma_tile = [&](const uint8_t* src, uint8_t* dst, int key0, bool is_v) {
#pragma unroll
      for (int u = 0; u < IPW; ++u) {
        const int row0 = RPI * (wq * IPW + u);
        const int row = row0 + lane / CH;
        const int phys = lane % CH;
        const int swz = is_v ? 2 * (row & 3) : (row & 7);
        const int key = min(key0 + row, p.S - 1);
        __builtin_amdgcn_global_load_lds(src + (size_t)key * ROWB + 16 * (phys ^ swz),
                                         LDS_AS(void, dst + row0 * ROWB), 16, 0, 0);
      }
    };
    u32x4 kreg[ROPE ? 2 * PAIRS : 1];
    auto load_k_regs = [&](int key0) {
      const int key = min(key0 + kr, p.S - 1);
#pragma unroll
      for (int u = 0; u < PAIRS; ++u) {
        const int c = kj + 4 * u;
        kreg[2 * u] = ldg16(kg + (size_t)key * ROWB + 16 * c);
        kreg[2 * u + 1] = ldg16(kg + (size_t)key * ROWB + 16 * (c + CH / 2));
      }
    };
    // angle of (position t*BN + r, frequency i) in revolutions:
    //   frac(t*BN*f_i) + r*f_i, f_i = theta^(-2i/D) / (2 pi); the fraction of the
    //   tile's base angle is taken in fp64 so that it stays exact at long contexts
    auto rope_base_fill = [&](int t, int slot) {
      if (wq == 0 && lane < HALF) {
        const double rev = (double)(t * BN) * p.rope_frev[lane];
        rope_base[half][slot][lane] = (float)(rev - floor(rev));
        rope_base[half][slot][HALF + lane] = (float)p.rope_frev[lane];
      }
    };
    auto rotate_store_k = [&](uint8_t* dst, int slot) {
#pragma unroll
      for (int u = 0; u < PAIRS; ++u) {
        const int c = kj + 4 * u;
        u32x4 lo = kreg[2 * u], hi = kreg[2 * u + 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float r1[2], r2[2];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int i = 8 * c + 2 * e + s;
            // revolutions in [0, 1 + 64 f_i): v_sin/v_cos take revolutions directly
            const float rev = fmaf((float)kr, rope_base[half][slot][HALF + i], rope_base[half][slot][i]);
            const float cs = __builtin_amdgcn_cosf(rev);
            const float sn = __builtin_amdgcn_sinf(rev);
            const float x1 = Tag::to_f32(s ? (lo[e] >> 16) : (lo[e] & 0xffff));
            const float x2 = Tag::to_f32(s ? (hi[e] >> 16) : (hi[e] & 0xffff));
            r1[s] = x1 * cs - x2 * sn;
            r2[s] = x2 * cs + x1 * sn;
          }
          lo[e] = Tag::pack2(r1[0], r1[1]);
          hi[e] = Tag::pack2(r2[0], r2[1]);
        }
        *reinterpret_cast<u32x4*>(dst + kr * ROWB + 16 * (c ^ (kr & 7))) = lo;
        *reinterpret_cast<u32x4*>(dst + kr * ROWB + 16 * ((c + CH / 2) ^ (kr & 7))) = hi;
      }
    };

    // ---- prologue: tile t(0) = half into stage 0 ----
    if (half < n_kt) {
      dma_tile(vg, hbuf + TILEB, half * BN, true);
      if (ROPE) load_k_regs(half * BN);
      else dma_tile(kg, hbuf, half * BN, false);
    }
    if (ROPE) {
      rope_base_fill(half, 0);
      rope_base_fill(half + 2, 1);
      __syncthreads();
      if (half < n_kt) rotate_store_k(hbuf, 0);
    }

    f32x16 acc_o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
    float m_ref = kNegInf;  // exponent reference (scaled log2 domain), same in both lanes of a row
    float l_run = 0.f;      // sum over this lane's keys of exp2(s - m_ref)

#pragma unroll 1
    for (int i = 0; i < n_it; ++i) {
      const int t = 2 * i + half;
      const int st = i & 1;
      __builtin_amdgcn_s_waitcnt(0x3f70);  // this thread's direct loads have landed (vmcnt 0)
      __syncthreads();
      const int tn = t + 2;
      const bool has_next = (i + 1 < n_it) && (tn < n_kt);
      if (has_next) {
        dma_tile(vg, hbuf + ((st ^ 1) * 2 + 1) * TILEB, tn * BN, true);
        if (ROPE) load_k_regs(tn * BN);
        else dma_tile(kg, hbuf + (st ^ 1) * 2 * TILEB, tn * BN, false);
      }
      if (ROPE && i + 2 < n_it) rope_base_fill(t + 4, st);

      const int key0 = t * BN;
      const bool active = (t < n_kt) && !(CAUSAL && key0 > pw0 + 31);
      if (active) {
        const uint8_t* kb = hbuf + st * 2 * TILEB;
        const uint8_t* vb = kb + TILEB;
        // ---- S^T = K Q^T ----
        f32x16 acc_s[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          acc_s[nb] = f32x16{};
          const int row = 32 * nb + m;
          const uint8_t* krow = kb + row * ROWB;
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(krow + 16 * ((2 * kk + hh) ^ (row & 7)));
            const u32x4 bq = {qf[4 * kk], qf[4 * kk + 1], qf[4 * kk + 2], qf[4 * kk + 3]};
            acc_s[nb] = Tag::mfma32(a, bq, acc_s[nb]);
          }
        }
        // ---- mask, lazy online softmax ----
        const bool need_mask = (key0 + BN > p.S) || (CAUSAL && key0 + BN - 1 > pw0);
        if (need_mask) {
          // key = key0 + 4 hh + off(nb, r) is visible iff key <= min(qpos, S - 1)
          const int lim = (CAUSAL ? min(qpos, p.S - 1) : p.S - 1) - key0 - 4 * hh;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * nb + 8 * (r >> 2) + (r & 3) > lim) acc_s[nb][r] = kNegInf;
        }
        float mx = kNegInf;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc_s[nb][r]);
        mx = pair_max32(mx) * p.scale_log2;
        if (__ballot(mx > m_ref + kLazy)) {
          const float m_new = fmaxf(m_ref, mx);
          const float alpha = fast_exp2(m_ref - m_new);  // 0 when m_ref = -inf
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
          m_ref = m_new;
        }
        const float m_use = m_ref == kNegInf ? 0.f : m_ref;
        uint32_t pf[4][4];
        float psum = 0.f;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float e0 = fast_exp2(fmaf(acc_s[nb][r], p.scale_log2, -m_use));
            const float e1 = fast_exp2(fmaf(acc_s[nb][r + 1], p.scale_log2, -m_use));
            psum += e0 + e1;
            pf[2 * nb + (r >> 3)][(r & 7) >> 1] = Tag::pack2(e0, e1);
          }
        l_run += psum;
        // ---- O^T += V^T P^T (V^T via transposing LDS reads) ----
        const int g = lane >> 4, rr = lane & 15;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = 32 * db + 16 * (g & 1) + 4 * (rr & 3);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int tok1 = 16 * c + 4 * (g >> 1) + (rr >> 2), tok2 = tok1 + 8;
            const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(v4i16,
                vb + tok1 * ROWB + 16 * ((d >> 3) ^ (2 * (tok1 & 3))) + 2 * (d & 7)));
            const v4i16 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(v4i16,
                vb + tok2 * ROWB + 16 * ((d >> 3) ^ (2 * (tok2 & 3))) + 2 * (d & 7)));
            const u32x4 a = {(uint32_t)(uint16_t)x1[0] | ((uint32_t)(uint16_t)x1[1] << 16),
                             (uint32_t)(uint16_t)x1[2] | ((uint32_t)(uint16_t)x1[3] << 16),
                             (uint32_t)(uint16_t)x2[0] | ((uint32_t)(uint16_t)x2[1] << 16),
                             (uint32_t)(uint16_t)x2[2] | ((uint32_t)(uint16_t)x2[3] << 16)};
            const u32x4 bp = {pf[c][0], pf[c][1], pf[c][2], pf[c][3]};
            acc_o[db] = Tag::mfma32(a, bp, acc_o[db]);
          }
        }
      }
      if (ROPE && has_next) rotate_store_k(hbuf + (st ^ 1) * 2 * TILEB, (st ^ 1));
    }

    // ---- merge the two halves (same rows, disjoint key tiles) ----
    __syncthreads();
    float* sc = reinterpret_cast<float*>(smem) + wq * (NDB * 16 + 2) * 64;
    if (half == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[(db * 16 + r) * 64 + lane] = acc_o[db][r];
      sc[(NDB * 16) * 64 + lane] = m_ref;
      sc[(NDB * 16 + 1) * 64 + lane] = l_run;
    }
    __syncthreads();
    if (half == 0) {
      const float m1 = sc[(NDB * 16) * 64 + lane], l1 = sc[(NDB * 16 + 1) * 64 + lane];
      const float M = fmaxf(m_ref, m1);
      const float Mu = M == kNegInf ? 0.f : M;
      const float f0 = fast_exp2(m_ref - Mu), f1 = fast_exp2(m1 - Mu);
      const float l = pair_sum32(l_run * f0 + l1 * f1);
      const float inv = l > 0.f ? p.out_scale / l : 0.f;
      if (qpos < p.S) {
        const size_t obase = (((size_t)b * p.Hq + head) * p.S + qpos) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float v4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * g4 + e;
              v4[e] = (acc_o[db][r] * f0 + sc[(db * 16 + r) * 64 + lane] * f1) * inv;
            }
            store4(p.o, obase + 32 * db + 8 * g4 + 4 * hh, p.out_dtype, v4[0], v4[1], v4[2], v4[3]);
          }
        if (p.lse && hh == 0)
          p.lse[((size_t)b * p.Hq + head) * p.S + qpos] = l > 0.f ? (Mu + __log2f(l)) * kLn2 : kNegInf;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 SIMT kernel: one query row per thread, 64 rows per workgroup.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool ROPE>
__global__ __launch_bounds__(64) void prefill_f32_kernel(const PrefillParams p) {
  constexpr int BN = 32;
  constexpr int HALF = D / 2;
  __shared__ float ks[BN][D];
  __shared__ float vs[BN][D];
  const int tid = threadIdx.x;
  const int head = blockIdx.y, b = blockIdx.z;
  const int kvh = head / p.G;
  const int r0 = blockIdx.x * 64;
  const int qpos = r0 + tid;
  const float* qsrc = reinterpret_cast<const float*>(p.q) + (((size_t)b * p.Hq + head) * p.S + min(qpos, p.S - 1)) * D;
  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { q[d] = qsrc[d]; o[d] = 0.f; }
  if (ROPE) {
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      float sn, cs;
      sincosf((float)qpos * p.inv_freq[i], &sn, &cs);
      const float x1 = q[i], x2 = q[i + HALF];
      q[i] = x1 * cs - x2 * sn;
      q[i + HALF] = x2 * cs + x1 * sn;
    }
  }
  const int kend = CAUSAL ? min(p.S, r0 + 64) : p.S;
  const float* kbase = reinterpret_cast<const float*>(p.k) + ((size_t)b * p.Hkv + kvh) * p.S * D;
  const float* vbase = reinterpret_cast<const float*>(p.v) + ((size_t)b * p.Hkv + kvh) * p.S * D;
  float m_run = kNegInf, l_run = 0.f;
  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    for (int e = tid; e < BN * D; e += 64) {
      const int r = e / D, d = e % D;
      const int key = k0 + r;
      ks[r][d] = key < p.S ? kbase[(size_t)key * D + d] : 0.f;
      vs[r][d] = key < p.S ? vbase[(size_t)key * D + d] : 0.f;
    }
    if (ROPE) {
      __syncthreads();
      for (int e = tid; e < BN * HALF; e += 64) {
        const int r = e / HALF, i = e % HALF;
        float sn, cs;
        sincosf((float)(k0 + r) * p.inv_freq[i], &sn, &cs);
        const float x1 = ks[r][i], x2 = ks[r][i + HALF];
        ks[r][i] = x1 * cs - x2 * sn;
        ks[r][i + HALF] = x2 * cs + x1 * sn;
      }
    }
    __syncthreads();
    float s[BN];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(q[d], ks[j][d], acc);
      const int key = k0 + j;
      s[j] = (key >= p.S || (CAUSAL && key > qpos)) ? kNegInf : acc * p.scale_log2;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const float pj = exp2f(s[j] - m_use);
      l_run += pj;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(pj, vs[j][d], o[d]);
    }
  }
  if (qpos < p.S) {
    const float inv = l_run > 0.f ? p.out_scale / l_run : 0.f;
    const size_t obase = (((size_t)b * p.Hq + head) * p.S + qpos) * D;
#pragma unroll
    for (int d = 0; d < D; d += 4) store4(p.o, obase + d, p.out_dtype, o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
    if (p.lse) p.lse[((size_t)b * p.Hq + head) * p.S + qpos] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Host dispatch
// ---------------------------------------------------------------------------
template <class Tag, int D>
static void launch_v2(const PrefillParams& p, bool causal, bool rope, hipStream_t st) {
  const long long items = (long long)p.n_ptiles * p.B * p.Hkv * p.n_hgroups;
  const dim3 grid((unsigned)(causal ? (items + 1) / 2 : items));
  if (causal) {
    if (rope) hipLaunchKernelGGL((prefill_v2_kernel<Tag, D, true, true>), grid, dim3(512), 0, st, p);
    else hipLaunchKernelGGL((prefill_v2_kernel<Tag, D, true, false>), grid, dim3(512), 0, st, p);
  } else {
    if (rope) hipLaunchKernelGGL((prefill_v2_kernel<Tag, D, false, true>), grid, dim3(512), 0, st, p);
    else hipLaunchKernelGGL((prefill_v2_kernel<Tag, D, false, false>), grid, dim3(512), 0, st, p);
  }
}

template <class Tag, int D, bool FP8>
static void launch_mfma(const PrefillParams& p, bool causal, dim3 grid, hipStream_t st) {
  if (causal) hipLaunchKernelGGL((prefill_mfma_kernel<Tag, D, true, false, FP8>), grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL((prefill_mfma_kernel<Tag, D, false, false, FP8>), grid, dim3(256), 0, st, p);
}

template <int D>
static void launch_f32(const PrefillParams& p, bool causal, bool rope, hipStream_t st) {
  dim3 grid((p.S + 63) / 64, p.Hq, p.B);
  if (causal) {
    if (rope) hipLaunchKernelGGL((prefill_f32_kernel<D, true, true>), grid, dim3(64), 0, st, p);
    else hipLaunchKernelGGL((prefill_f32_kernel<D, true, false>), grid, dim3(64), 0, st, p);
  } else {
    if (rope) hipLaunchKernelGGL((prefill_f32_kernel<D, false, true>), grid, dim3(64), 0, st, p);
    else hipLaunchKernelGGL((prefill_f32_kernel<D, false, false>), grid, dim3(64), 0, st, p);
  }
}

}  // namespace attn

using namespace attn;

extern "C" attn_status attn_prefill_gqa_rope(const void* q, const void* k, const void* v, void* o,
                                             float* lse, int B, int Hq, int Hkv, int S, int D,
                                             attn_dtype in_dtype, attn_dtype out_dtype,
                                             float softmax_scale, int causal, float rope_theta,
                                             float q_descale, float k_descale, float v_descale,
                                             hipStream_t stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (in_dtype < ATTN_F32 || in_dtype > ATTN_FP8_E5M2) return ATTN_ERR_DTYPE;
  if (out_dtype != ATTN_F32 && out_dtype != ATTN_F16 && out_dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  // the score scale must be a positive finite number (the kernels take row maxima of raw scores)
  const float sc_all = softmax_scale * q_descale * k_descale;
  if (!(sc_all > 0.f) || !(sc_all < 3.0e38f) || !(v_descale == v_descale)) return ATTN_ERR_SHAPE;
  const bool rope = rope_theta > 0.f;
  if (rope && in_dtype == ATTN_FP8_E5M2) return ATTN_ERR_UNSUPPORTED;
  if (!attn_host::aligned(q, 16) || !attn_host::aligned(k, 16) || !attn_host::aligned(v, 16) ||
      !attn_host::aligned(o, 16) || (lse && !attn_host::aligned(lse, 4)))
    return ATTN_ERR_ALIGN;
  // sizes: element offsets fit comfortably in 64-bit; keep grid item counts in int range
  const long long elems_q = (long long)B * Hq * S * D;
  if (elems_q > (1LL << 40)) return ATTN_ERR_SHAPE;

  PrefillParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.S = S;
  p.G = Hq / Hkv;
  p.scale_log2 = softmax_scale * q_descale * k_descale * kLog2e;
  p.out_scale = v_descale;
  p.out_dtype = out_dtype;
  p.rope = rope ? 1 : 0;
  for (int i = 0; i < D / 2; ++i) {
    const double w = rope ? pow((double)rope_theta, -2.0 * i / D) : 0.0;
    p.inv_freq[i] = (float)w;
    p.rope_frev[i] = w / (2.0 * 3.14159265358979323846);
  }

  if (in_dtype == ATTN_F32) {
    p.GP = 1; p.P = 64; p.n_ptiles = (S + 63) / 64; p.n_hgroups = p.G;
    if ((long long)p.n_ptiles > 65535 || Hq > 65535 || B > 65535) return ATTN_ERR_SHAPE;
    if (D == 64) launch_f32<64>(p, causal != 0, rope, stream);
    else launch_f32<128>(p, causal != 0, rope, stream);
    return attn_host::launch_status();
  }

  // heads of one KV group per workgroup: the largest of 4, 2, 1 dividing G
  p.GP = (p.G % 4 == 0) ? 4 : (p.G % 2 == 0) ? 2 : 1;
  p.P = 128 / p.GP;
  p.n_ptiles = (S + p.P - 1) / p.P;
  p.n_hgroups = p.G / p.GP;
  const long long items = (long long)p.n_ptiles * B * Hkv * p.n_hgroups;
  if (items > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  dim3 grid((unsigned)items);
  const bool c = causal != 0;
  switch (in_dtype) {
    case ATTN_BF16:
      if (D == 64) launch_v2<Bf16Tag, 64>(p, c, rope, stream);
      else launch_v2<Bf16Tag, 128>(p, c, rope, stream);
      break;
    case ATTN_F16:
      if (D == 64) launch_v2<F16Tag, 64>(p, c, rope, stream);
      else launch_v2<F16Tag, 128>(p, c, rope, stream);
      break;
    default:  // fp8 e5m2 (RoPE rejected above)
      if (D == 64) launch_mfma<F16Tag, 64, true>(p, c, grid, stream);
      else launch_mfma<F16Tag, 128, true>(p, c, grid, stream);
      break;
  }
  return attn_host::launch_status();
}
