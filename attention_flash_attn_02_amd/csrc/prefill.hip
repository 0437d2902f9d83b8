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

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "prefill_common.hpp"
#include "rope_common.hpp"

namespace attn {

template <int N>
using ic_t = std::integral_constant<int, N>;



// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------
// P8 (fp8 inputs): PV on the fp8 MFMA with P rounded to e4m3 and V^T staged
// as its e5m2 bytes (twice the f16 MFMA rate); the row sums are taken by the
// same MFMA against a matrix of ones, so they add up exactly the rounded
// probabilities that weight V.
// (launch bounds of two waves per SIMD: unbounded, the allocator took 236-276
// registers and one wave per SIMD; bounded, 125-188 without spills, and the
// fp8 forward runs 10-50 % faster)
template <class Tag, int D, bool CAUSAL, bool ROPE, bool FP8, bool P8 = false>
__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(const PrefillParams p) {
  static_assert(!P8 || FP8, "e4m3 P needs fp8 inputs");
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
  constexpr int V8PITCH = 80;            // bytes per V^T row in LDS (P8; 5 x 16 keeps reads conflict-free)
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[P8 ? 1 : D * VPITCH];
  __shared__ __attribute__((aligned(16))) uint8_t v8_lds[P8 ? D * V8PITCH : 1];
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
    // ---- V -> LDS, transposed ----
    if constexpr (P8) {
      // e5m2 bytes: v8_lds[d][32 h + j] holds key 32 (j / 16) + 8 ((j % 16) / 4)
      // + 4 h + j % 4, the order in which lane half h holds its 32 keys in
      // the score accumulator (so P^T packs straight from registers)
      const int posv = 32 * ((vn0 >> 2) & 1) + 16 * (vn0 >> 5) + 4 * ((vn0 >> 3) & 3) + (vn0 & 3);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t wv = 0;
#pragma unroll
        for (int r = 0; r < KPT; ++r) wv |= ((vbuf8[r][i >> 2] >> (8 * (i & 3))) & 0xffu) << (8 * r);
        uint8_t* dst = v8_lds + (8 * vdc + i) * V8PITCH + posv;
        if (KPT == 4) *reinterpret_cast<uint32_t*>(dst) = wv;
        else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)wv;
      }
      return;
    }
    // ---- v_lds[d][pos] (16-bit) ----
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
  f32x16 acc_l = f32x16{};  // P8: row sums of the rounded probabilities (every row of a column equal)
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
    if constexpr (P8) {
      // P^T as e4m3, k order j = 16 nb + i (the accumulator's order)
      i32x8 pb;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int nb = w >> 2, i0 = 4 * (w & 3);
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(fast_exp2(acc_s[nb][i0] - m_use), fast_exp2(acc_s[nb][i0 + 1] - m_use), 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(fast_exp2(acc_s[nb][i0 + 2] - m_use), fast_exp2(acc_s[nb][i0 + 3] - m_use), v, true);
        pb[w] = v;
      }
      acc_l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
      const i32x8 ones = {0x3c3c3c3c, 0x3c3c3c3c, 0x3c3c3c3c, 0x3c3c3c3c,
                          0x3c3c3c3c, 0x3c3c3c3c, 0x3c3c3c3c, 0x3c3c3c3c};  // e5m2 1.0
      acc_l = mfma32_bf8_fp8(ones, pb, acc_l);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint8_t* vrow = v8_lds + (32 * db + m) * V8PITCH + 32 * hh;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(vrow), a1 = *reinterpret_cast<const u32x4*>(vrow + 16);
        const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        acc_o[db] = mfma32_bf8_fp8(a, pb, acc_o[db]);
      }
      continue;
    }
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
  const float l_tot = P8 ? acc_l[0] : l_run + __shfl_xor(l_run, 32);
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

// chunk mode with several key ranges: the ranges' parts in bf16 (1) or fp32 (0)
#ifndef ATTN_CHUNK_BF16_PARTS
#define ATTN_CHUNK_BF16_PARTS 1
#endif
// cache policy of the chunk-mode row stores (16: sc1, device scope)
#ifndef ATTN_CHUNK_OAUX
#define ATTN_CHUNK_OAUX 16
#endif

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
// One workgroup barrier per key tile: after it, each half issues the loads of
// its next tile into the other LDS stage and computes S^T = K Q^T, the online
// softmax and O^T += V^T P^T for its current tile.  MFMA operands are read
// from LDS a few MFMAs ahead of their use.
//
// K and V tiles go straight from HBM to LDS (buffer loads with the LDS bit, 16 B per lane)
// into XOR-swizzled row-major layouts, two stages per tensor per half.  V is
// read transposed by ds_read_b64_tr_b16: each 16-lane group reads a 4-key x
// 16-dim block and every lane receives one dim column of 4 keys, which is
// exactly the A operand of O^T = V^T P^T.  With RoPE the K tile is loaded
// into registers, rotated in a V-step and written to LDS.  The running row
// maximum is only moved when a row's maximum exceeds it by more than 2^8
// (lazy rescaling: exact, the probabilities just stay below 256).
// ---------------------------------------------------------------------------
// CHUNK: the queries are a chunk of p.S rows at the end of a cache prefix:
// K/V rows come from caches with p.cap slots per head, the key length of
// sequence b is kv_len[b] (read on the device) and query row r sits at
// position kv_len[b] - p.S + r (causal with that offset).  With RoPE (mode
// 2) the Q rows are rotated here to those positions; the cached K rows were
// rotated when they were appended.
// PERSIST: resident workgroups loop over several items (see below).
// BNT: keys per tile.  64 by default; 32 halves the LDS of a workgroup
// (three workgroups, i.e. three waves per SIMD, fit a compute unit) and the
// score registers, for the plain 4-wave kernel with K moved by DMA.
// PP (8-wave workgroups only): the halves' waves share SIMDs pairwise, and
// with one barrier per key tile they would run the same phase at the same
// time (both on the matrix cores, then both on the softmax ALU work).  With
// PP each key tile has two barriers, one after the S MFMAs and one before
// the PV MFMAs, and the second half passes one extra barrier before its key
// loop (the first half one after it).  Every barrier instance then finds one
// half between its two barriers (the softmax of a tile) and the other half
// between the second and the next first (the PV MFMAs of a tile and the S
// MFMAs of the next), so softmax work and MFMAs of the two halves overlap.
// Each half's 4 waves still meet at one program point per instance, and each
// half stages its own tiles, so the LDS protocol holds within each half: K
// runs one tile ahead of V; each wave waits for its loads of V of tile i and
// K of tile i+1 before the second barrier of tile i, and after its PV MFMAs
// of tile i issues V of tile i+1 and K of tile i+2 into the stages of V(i-1)
// and K(i), which every wave of the half finished reading before that
// barrier.
// RS (4-wave workgroups only): K and V tiles go HBM -> registers -> LDS
// (buffer loads after the loop-top barrier, swizzled LDS stores after the PV
// MFMAs) instead of by DMA.  The compiler makes every transposing LDS read
// wait for all LDS DMA in flight (`vmcnt(0)`), so with DMA the PV MFMAs of a
// tile wait for the next tile's loads; register loads are waited for only
// where their registers are stored.
template <class Tag, int D, bool CAUSAL, int ROPE, int HALVES, bool CHUNK = false, bool PERSIST = false, int BNT = 64,
          bool PP = false, bool RS = false>
__global__ __launch_bounds__(256 * HALVES, BNT == 32 ? 3 : 2) void prefill_fwd_kernel(const PrefillParams p) {
  static_assert(!CHUNK || (CAUSAL && ROPE != 1 && HALVES == 1), "chunk mode: causal, K already rotated, 4 waves");
  static_assert(!PERSIST || (HALVES == 1 && !CHUNK), "persistent scheduling: 4 waves, plain prefill");
  static_assert(BNT == 64 || (BNT == 32 && ROPE != 1 && HALVES == 1 && !CHUNK && !PERSIST),
                "32-key tiles: plain 4-wave kernel with K moved by DMA");
  static_assert(!PP || (HALVES == 2 && ROPE != 1 && !CHUNK && !PERSIST && BNT == 64),
                "offset halves: 8-wave kernel with K moved by DMA");
  static_assert(!RS || (HALVES == 1 && ROPE != 1 && !CHUNK && !PERSIST && BNT == 64 && !PP),
                "register-staged tiles: plain 4-wave kernel");
  constexpr int BN = BNT;
  constexpr int NB = BN / 32;   // 32-key blocks of the score tile
  constexpr int CPB = BN / 16;  // 16-key k-steps of the PV MFMAs
  constexpr int ROWB = D * 2;        // bytes per K/V row
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int TILEB = BN * ROWB;   // bytes of one K or V tile
  constexpr int RPI = 64 / CH;       // rows per wave-wide direct load
  constexpr int IPW = BN / RPI / 4;  // direct loads per wave per tile
  constexpr int NKK = D / 16, NDB = D / 32, HALF = D / 2, PAIRS = D / 64;
  constexpr float kLazy = 8.f;
  // RoPE mode: 0 none; 1 Q and K rotated here (K tiles while they are staged);
  // 2 Q rotated here, K already rotated in HBM
  constexpr bool RQ = ROPE != 0, RK = ROPE == 1;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[HALVES * 4 * TILEB];  // [half][K0 K1 V0 V1]
  __shared__ float rope_base[2][2][RK ? D : 1];                          // [half][slot][rev0 | freq]

  // XOR swizzles of the 16-byte chunks of a row, for a 64-bank LDS (one
  // 256-byte bank line = one D=128 row or two D=64 rows):
  //   K, read by 16 consecutive rows at one chunk: rows must hit 16 distinct
  //   bank groups;  V, read transposed as 4 rows x 4 chunks per 32 lanes.
  auto kswz = [](int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); };
  auto vswz = [](int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); };
  // (8 waves and chunk mode: the wave index is read into a scalar register,
  // so that the tile addresses are wave-uniform and the buffer loads take
  // scalar descriptors directly instead of a loop over the distinct values;
  // the plain 4-wave kernel measured slower that way and keeps tid >> 6)
  const int tid = threadIdx.x, wave = (HALVES == 2 || CHUNK) ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int lane = tid & 63;
  const int half = HALVES == 2 ? wave >> 2 : 0, wq = wave & 3, htid = tid & 255;
  const int m = lane & 31, hh = lane >> 5;
  const int g = lane >> 4, rr = lane & 15;
  uint8_t* hbuf = smem + half * (4 * TILEB);

  // ---- lane-constant LDS offsets ----
  // K A operand: row 32 nb + m (the swizzle depends on m only), logical chunk 2 kk + hh
  int koff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) koff[kk] = m * ROWB + 16 * ((2 * kk + hh) ^ kswz(m));
  // V^T A operand via transposing reads: this lane addresses key
  // 16 c + 4 (g >> 1) + (rr >> 2) (+ 8), dims 32 db + 16 (g & 1) + 4 (rr & 3) .. + 3
  // (the swizzle only depends on key mod 4, which the offsets 16 c and 8 keep)
  int voff[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d = 32 * db + 16 * (g & 1) + 4 * (rr & 3);
    const int key = 4 * (g >> 1) + (rr >> 2);
    voff[db] = key * ROWB + 16 * ((d >> 3) ^ vswz(key)) + 2 * (d & 7);
  }
  // direct-load lane offsets (row inside the tile, swizzled source chunk)
  int dk[IPW], dv[IPW];
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int row = RPI * (wq * IPW + u) + lane / CH, phys = lane % CH;
    dk[u] = row * ROWB + 16 * (phys ^ kswz(row));
    dv[u] = row * ROWB + 16 * (phys ^ vswz(row));
  }

  // chunk mode is latency-bound: have every kernel argument the item set-up
  // reads arrive in one batch of scalar loads (left to themselves, the loads
  // are issued at first use, one dependent round trip after another)
  if constexpr (CHUNK)
    asm volatile("" ::"s"(p.B), "s"(p.Hkv), "s"(p.n_hgroups), "s"(p.n_ptiles), "s"(p.nsplit), "s"(p.G), "s"(p.GP),
                 "s"(p.P), "s"(p.S), "s"(p.Hq), "s"(p.q), "s"(p.k_new), "s"(p.v_new), "s"(p.k), "s"(p.v),
                 "s"(p.cap), "s"(p.split_keys), "s"(p.kv_len));
  const int per_ptile = p.B * p.Hkv * p.n_hgroups;
  // (chunk mode: every item is further split into p.nsplit key ranges)
  const int n_items = p.n_ptiles * per_ptile * (CHUNK ? p.nsplit : 1);
  // causal, 8 waves: this workgroup takes long item k and short item n-1-k.
  // 4 waves: one item; the second half of the grid takes the short items in
  // reverse order, so that workgroups k and k + n/2 (which tend to share a CU
  // when two workgroups fit per CU) carry complementary amounts of work.
  const int half_items = (n_items + 1) / 2;
  int item_long = blockIdx.x, item_short = n_items - 1 - (int)blockIdx.x;
  if (HALVES == 1 && CAUSAL)
    item_long = (int)blockIdx.x < half_items ? (int)blockIdx.x : n_items - 1 - ((int)blockIdx.x - half_items);
  // persistent scheduling (4 waves): gridDim.x resident workgroups walk the
  // longest-first item list in snake order, round k taking item
  // k W + w (k even) or k W + W - 1 - w (k odd), so that every workgroup
  // gets a balanced mix of long and short items
  constexpr bool persist = PERSIST;
  const int n_my = persist ? (n_items + (int)gridDim.x - 1) / (int)gridDim.x
                           : (HALVES == 2 && CAUSAL && item_short > item_long) ? 2 : 1;
  // RoPE staging: row kr, chunk pairs (kj + 4u, + CH/2); 16 consecutive lanes
  // take 16 rows at one chunk so the LDS writes hit 16 distinct bank groups
  const int kr = (htid & 15) + 16 * (htid >> 6), kj = (htid >> 4) & 3;
  // frequency lane of the per-tile angle table, read from the kernel
  // arguments once (not inside the key loop, where the load latency would
  // hold up the filling wave every tile)
  const float fhi_lane = RK && lane < HALF ? p.rope_fhi[lane] : 0.f;
  const float flo_lane = RK && lane < HALF ? p.rope_flo[lane] : 0.f;
  // cos / sin of the row-offset angles kr f_j of this thread's K pairs
  // (kr < 64 and f_hi has 8 significant bits, so kr f_hi is exact)
  float rcos[RK ? 8 * PAIRS : 1], rsin[RK ? 8 * PAIRS : 1];
  if (RK) {
#pragma unroll
    for (int u = 0; u < PAIRS; ++u)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int j = 8 * (kj + 4 * u) + t;
        const float rev = __builtin_amdgcn_fractf((float)kr * p.rope_fhi[j]) + (float)kr * p.rope_flo[j];
        rcos[8 * u + t] = __builtin_amdgcn_cosf(rev);
        rsin[8 * u + t] = __builtin_amdgcn_sinf(rev);
      }
  }

#pragma unroll 1
  for (int itn = 0; itn < n_my; ++itn) {
    if (itn > 0) __syncthreads();  // LDS of the previous item is free
    const int item_ks = persist ? itn * (int)gridDim.x + ((itn & 1) ? (int)gridDim.x - 1 - (int)blockIdx.x
                                                                    : (int)blockIdx.x)
                                : itn == 0 ? item_long : item_short;
    if (item_ks >= n_items) break;  // (persistent: uniform over the workgroup)
    const int split = CHUNK ? item_ks % p.nsplit : 0;  // key range of this item
    const int item = CHUNK ? item_ks / p.nsplit : item_ks;
    const int ptile = p.n_ptiles - 1 - item / per_ptile;
    int rest = item % per_ptile;
    const int hg = rest % p.n_hgroups;
    rest /= p.n_hgroups;
    const int kvh = rest % p.Hkv;
    const int b = rest / p.Hkv;
    const int head = kvh * p.G + hg * p.GP + (wq % p.GP);
    const int p0 = ptile * p.P;
    const int pw0 = p0 + (wq / p.GP) * 32;
    // Q rows (B operand of S^T = K Q^T), loaded unrotated; in chunk mode
    // before the key length is read, so that the two loads overlap
    uint32_t qf[D / 4];
    auto load_q = [&]() {
      const int qp = pw0 + m;
      const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + (((size_t)b * p.Hq + head) * p.S + min(qp, p.S - 1)) * D;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const u32x4 w = ldg16(qrow + 16 * kk + 8 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[4 * kk + e] = w[e];
      }
    };
    // chunk mode that appends: this thread's share of the chunk's K (chunk
    // pairs) and V (chunks) rows, loaded with the query rows, before the key
    // length is known
    constexpr int ACPR = D / 16, ACPF = D / 8;  // 16-byte chunk pairs / chunks per 16-bit row
    constexpr int AKU = (32 * ACPR + 255) / 256, AVU = (32 * ACPF + 255) / 256;
    const bool app = CHUNK && p.k_new != nullptr;
    u32x4 ak[CHUNK ? AKU : 1][2], av[CHUNK ? AVU : 1];
    // chunk mode: the key length is read first; its round trip overlaps the
    // loads below, none of which depends on it
    int lkv_read = 0;
    if (CHUNK) {
      lkv_read = p.kv_len[b];
      __builtin_amdgcn_sched_barrier(0);
      load_q();
      if (app) {
        const size_t nrow0 = ((size_t)b * p.Hkv + kvh) * p.S;
        const uint8_t* kn = reinterpret_cast<const uint8_t*>(p.k_new) + nrow0 * ROWB;
        const uint8_t* vn = reinterpret_cast<const uint8_t*>(p.v_new) + nrow0 * ROWB;
#pragma unroll
        for (int u = 0; u < AKU; ++u) {
          const int w = htid + 256 * u, t = min(w / ACPR, p.S - 1), c = w % ACPR;
          ak[u][0] = ldg16(kn + (size_t)t * ROWB + 16 * c);
          ak[u][1] = ldg16(kn + (size_t)t * ROWB + D + 16 * c);
        }
#pragma unroll
        for (int u = 0; u < AVU; ++u) {
          const int w = htid + 256 * u, t = min(w / ACPF, p.S - 1), c = w % ACPF;
          av[u] = ldg16(vn + (size_t)t * ROWB + 16 * c);
        }
      }
      // tile 0 of this item's key range, before the key length is known:
      // its address does not depend on it.  The buffer range ends at the
      // capacity instead of the key length, so the rows from the key length
      // on hold what the cache held when the load read them; they are fixed
      // in LDS below, before any use.
      {
        const int kb0 = split * p.split_keys;
        const size_t row0 = ((size_t)b * p.Hkv + kvh) * p.cap + kb0;
        const int range = max(0, p.cap - kb0) * ROWB;
        auto early_dma = [&](const void* base, uint8_t* dst, const int* loff) {
          const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(base) + row0 * ROWB), (short)0, range,
              kBufferRsrcWord3);
#pragma unroll
          for (int u = 0; u < IPW; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_AS(void, dst + RPI * (wq * IPW + u) * ROWB), 16, loff[u], 0, 0, 0);
        };
        early_dma(p.k, hbuf, dk);
        early_dma(p.v, hbuf + 2 * TILEB, dv);
      }
      __builtin_amdgcn_sched_barrier(0);  // (the scheduler would otherwise wait for the key length first)
    }
    // key length and query position offset (plain prefill: S and 0)
    // (moved to a scalar register only here: converted at the load, the
    // value would be waited for before the loads above were issued)
    const int Lkv = CHUNK ? max(__builtin_amdgcn_readfirstlane(lkv_read), 0) : 0;
    const int Skv = CHUNK ? min(Lkv + p.kv_add, p.cap) : p.S;
    const int qoff = CHUNK ? Skv - p.S : 0;
    const int kend_all = CAUSAL ? max(0, min(Skv, qoff + p0 + p.P)) : Skv;
    // key range [kbeg, kend) of this item: all keys, or (chunk mode) split
    // `split` of p.split_keys keys (a multiple of the 64-key tile)
    const int kbeg = CHUNK ? split * p.split_keys : 0;
    const int kend = CHUNK ? min(kend_all, kbeg + p.split_keys) : kend_all;
    const int t0 = kbeg / BN;  // first key tile
    const int n_kt = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;
    const int n = (n_kt + HALVES - 1) / HALVES;  // local tiles per half: local i is tile HALVES i + half
    const int qpos = pw0 + m;

    const size_t kv_row0 = ((size_t)b * p.Hkv + kvh) * (CHUNK ? p.cap : p.S);
    const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.k) + kv_row0 * ROWB;
    const uint8_t* vg = reinterpret_cast<const uint8_t*>(p.v) + kv_row0 * ROWB;
    auto exists = [&](int i) { return i >= 0 && i < n && HALVES * i + half < n_kt; };
    auto kbuf = [&](int i) { return hbuf + (i & 1) * TILEB; };
    auto vbuf = [&](int i) { return hbuf + (2 + (i & 1)) * TILEB; };

    // direct HBM -> LDS load of local tile i of K or V.  The buffer resource
    // starts at the tile's first row and ends at row S, so rows past S read
    // as zero without a memory access (those keys are masked and their
    // probabilities are exactly 0); all address arithmetic is scalar.
    auto tile_rsrc = [&](const uint8_t* src, int i) {
      const int key0 = (t0 + HALVES * i + half) * BN;
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src + (size_t)key0 * ROWB), (short)0,
                                               (Skv - key0) * ROWB, kBufferRsrcWord3);
    };
    auto dma = [&](const uint8_t* src, uint8_t* dst, const int* loff, int i) {
      const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src, i);
#pragma unroll
      for (int u = 0; u < IPW; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_AS(void, dst + RPI * (wq * IPW + u) * ROWB), 16, loff[u], 0, 0, 0);
    };
    // register staging (RS): this wave's IPW 16-byte chunks of a K tile and
    // of a V tile, at the rows and chunks the DMA would move
    u32x4 sreg[RS ? 2 * IPW : 1];
    auto stage_load = [&](int i) {
      const __amdgpu_buffer_rsrc_t ks = tile_rsrc(kg, i), vs = tile_rsrc(vg, i);
#pragma unroll
      for (int u = 0; u < IPW; ++u) {
        const int off = (RPI * (wq * IPW + u) + lane / CH) * ROWB + 16 * (lane % CH);
        sreg[u] = __builtin_amdgcn_raw_buffer_load_b128(ks, off, 0, 0);
        sreg[IPW + u] = __builtin_amdgcn_raw_buffer_load_b128(vs, off, 0, 0);
      }
    };
    auto stage_store = [&](int i) {
#pragma unroll
      for (int u = 0; u < IPW; ++u) {
        const int row = RPI * (wq * IPW + u) + lane / CH, c = lane % CH;
        *reinterpret_cast<u32x4*>(kbuf(i) + row * ROWB + 16 * (c ^ kswz(row))) = sreg[u];
        *reinterpret_cast<u32x4*>(vbuf(i) + row * ROWB + 16 * (c ^ vswz(row))) = sreg[IPW + u];
      }
    };
    u32x4 kreg[RK ? 2 * PAIRS : 1];
    auto load_k_regs = [&](int i) {
      const __amdgpu_buffer_rsrc_t rs = tile_rsrc(kg, i);
#pragma unroll
      for (int u = 0; u < PAIRS; ++u) {
        const int c = kj + 4 * u;
        kreg[2 * u] = __builtin_amdgcn_raw_buffer_load_b128(rs, kr * ROWB + 16 * c, 0, 0);
        kreg[2 * u + 1] = __builtin_amdgcn_raw_buffer_load_b128(rs, kr * ROWB + 16 * (c + CH / 2), 0, 0);
      }
    };
    // RoPE angle of (position key0 + r, frequency j) = base angle of the tile
    // (key0 f_j, reduced exactly as frac(key0 f_hi) + key0 f_lo revolutions)
    // plus the row offset r f_j.  The table holds cos and sin of the base
    // angles of a tile; cos and sin of the row offsets are per-thread
    // constants, and the two are combined by the angle-addition formulas.
    auto rope_base_fill = [&](int i) {
      if (wq == 0 && lane < HALF) {
        const float key0 = (float)((t0 + HALVES * i + half) * BN);
        const float rev = __builtin_amdgcn_fractf(key0 * fhi_lane) + key0 * flo_lane;
        rope_base[half][i & 1][lane] = __builtin_amdgcn_cosf(rev);
        rope_base[half][i & 1][HALF + lane] = __builtin_amdgcn_sinf(rev);
      }
    };
    auto rotate_store_k = [&](int i) {
      uint8_t* dst = kbuf(i);
#pragma unroll
      for (int u = 0; u < PAIRS; ++u) {
        const int c = kj + 4 * u;
        u32x4 lo = kreg[2 * u], hi = kreg[2 * u + 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float r1[2], r2[2];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int j = 8 * c + 2 * e + s, t = 8 * u + 2 * e + s;
            const float cb = rope_base[half][i & 1][j], sb = rope_base[half][i & 1][HALF + j];
            const float cs = cb * rcos[t] - sb * rsin[t], sn = sb * rcos[t] + cb * rsin[t];
            const float x1 = Tag::to_f32(s ? (lo[e] >> 16) : (lo[e] & 0xffff));
            const float x2 = Tag::to_f32(s ? (hi[e] >> 16) : (hi[e] & 0xffff));
            r1[s] = x1 * cs - x2 * sn;
            r2[s] = x2 * cs + x1 * sn;
          }
          lo[e] = Tag::pack2(r1[0], r1[1]);
          hi[e] = Tag::pack2(r2[0], r2[1]);
        }
        *reinterpret_cast<u32x4*>(dst + kr * ROWB + 16 * (c ^ kswz(kr))) = lo;
        *reinterpret_cast<u32x4*>(dst + kr * ROWB + 16 * ((c + CH / 2) ^ kswz(kr))) = hi;
      }
    };
    auto active = [&](int i) {
      return exists(i) && !(CAUSAL && (t0 + HALVES * i + half) * BN > qoff + pw0 + 31);
    };

    // ---- chunk mode that appends: the chunk's rows of this item's key range
    //      go to the cache (K rotated to slot Lkv + t), and the workgroup
    //      waits for its stores before any wave loads them back (the loads
    //      of tiles 1, 2, ...); items of the same KV head and range write
    //      the same bytes.  Tile 0, loaded before the key length was known,
    //      then gets the chunk's rows that fall in it and zeros for the V
    //      rows past the key length (probability 0 times a non-finite value
    //      would not be 0; the keys there are masked). ----
    if (CHUNK) {
      const int key0 = kbeg;
      const bool fix0 = n_kt > 0 && Skv - key0 < BN;  // tile 0 ends past the key length
      const bool app0 = app && n_kt > 0 && Lkv < key0 + BN;  // ... or holds chunk rows
      if (app) {
        uint8_t* kcw = const_cast<uint8_t*>(kg);
        uint8_t* vcw = const_cast<uint8_t*>(vg);
#pragma unroll
        for (int u = 0; u < AKU; ++u) {
          const int w = htid + 256 * u, t = w / ACPR, c = w % ACPR, slot = Lkv + t;
          if (t < p.S && slot >= kbeg && slot < kend && slot < p.cap) {
            u32x4 lo = ak[u][0], hi = ak[u][1];
            if (ROPE == 2) rotate_chunk_pair<Tag>(lo, hi, (float)slot, c, p.rope_fhi, p.rope_fmid, p.rope_flo3);
            *reinterpret_cast<u32x4*>(kcw + (size_t)slot * ROWB + 16 * c) = lo;
            *reinterpret_cast<u32x4*>(kcw + (size_t)slot * ROWB + D + 16 * c) = hi;
            ak[u][0] = lo;
            ak[u][1] = hi;
          }
        }
#pragma unroll
        for (int u = 0; u < AVU; ++u) {
          const int w = htid + 256 * u, t = w / ACPF, c = w % ACPF, slot = Lkv + t;
          if (t < p.S && slot >= kbeg && slot < kend && slot < p.cap)
            *reinterpret_cast<u32x4*>(vcw + (size_t)slot * ROWB + 16 * c) = av[u];
        }
      }
      if (app || fix0) {
        __builtin_amdgcn_s_waitcnt(0);  // this thread's stores, and its share of tile 0
        __syncthreads();                // ... and everybody's
      }
      if (fix0 || app0) {
        if (fix0) {
          const int r0 = max(Skv - key0, 0);
#pragma unroll
          for (int u = 0; u < BN * CH / 256; ++u) {
            const int e = htid + 256 * u, r = e / CH, c = e % CH;
            if (r >= r0) *reinterpret_cast<u32x4*>(vbuf(0) + r * ROWB + 16 * c) = u32x4{0, 0, 0, 0};
          }
        }
        if (app0) {
#pragma unroll
          for (int u = 0; u < AKU; ++u) {
            const int w = htid + 256 * u, t = w / ACPR, c = w % ACPR, slot = Lkv + t;
            if (t < p.S && slot >= kbeg && slot < kend && slot < p.cap && slot < key0 + BN) {
              const int r = slot - key0;
              *reinterpret_cast<u32x4*>(kbuf(0) + r * ROWB + 16 * (c ^ kswz(r))) = ak[u][0];
              *reinterpret_cast<u32x4*>(kbuf(0) + r * ROWB + 16 * ((c + CH / 2) ^ kswz(r))) = ak[u][1];
            }
          }
#pragma unroll
          for (int u = 0; u < AVU; ++u) {
            const int w = htid + 256 * u, t = w / ACPF, c = w % ACPF, slot = Lkv + t;
            if (t < p.S && slot >= kbeg && slot < kend && slot < p.cap && slot < key0 + BN) {
              const int r = slot - key0;
              *reinterpret_cast<u32x4*>(vbuf(0) + r * ROWB + 16 * (c ^ vswz(r))) = av[u];
            }
          }
        }
        __syncthreads();
      }
    }

    // ---- running state ----
    f32x16 acc_o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
    float m_ref = kNegInf;  // exponent reference (scaled log2 domain), equal in both lanes of a row
    float l_run = 0.f;      // sum over this lane's keys of exp2(s - m_ref)

    // ---- prologue: local tile 0 into stage 0 ----
    if (RK) {
      rope_base_fill(0);
      rope_base_fill(1);
      if (exists(0)) {
        dma(vg, vbuf(0), dv, 0);
        load_k_regs(0);
      }
      __syncthreads();
      if (exists(0)) rotate_store_k(0);
    } else if (RS) {
      if (exists(0)) stage_load(0);
    } else if (exists(0) && !CHUNK) {  // (chunk mode: loaded above)
      dma(kg, kbuf(0), dk, 0);
      dma(vg, vbuf(0), dv, 0);
    }
    if (PP && exists(1)) dma(kg, kbuf(1), dk, 1);  // K runs one tile ahead of V

    // ---- Q fragments (B operand of S^T = K Q^T), loaded (and rotated) while
    //      the first tile's K/V loads are in flight ----
    {
      if (!CHUNK) {
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + (((size_t)b * p.Hq + head) * p.S + qpos) * D;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          u32x4 w = qpos < p.S ? ldg16(qrow + 16 * kk + 8 * hh) : u32x4{0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 4; ++e) qf[4 * kk + e] = w[e];
        }
      }
      if (RQ) {
#pragma unroll
        for (int kk = 0; kk < NKK / 2; ++kk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w1 = qf[4 * kk + e], w2 = qf[4 * (kk + NKK / 2) + e];
            float r1[2], r2[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              // angle in revolutions (v_sin/v_cos take revolutions)
              const int fi = 16 * kk + 8 * hh + 2 * e + s;
              const float pos = (float)(CHUNK ? max(qoff + qpos, 0) : qpos);
              const float rev = __builtin_amdgcn_fractf(pos * p.rope_fhi[fi]) + pos * p.rope_flo[fi];
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

    if (RS && exists(0)) stage_store(0);  // the loop-top barrier publishes it

    if constexpr (PP) {
      // the second half runs one barrier behind the first (see PP above);
      // `lag` is wave-uniform and held in a scalar register, so the extra
      // barriers are skipped by a scalar branch
      const bool lag = __builtin_amdgcn_readfirstlane(half) == 1;
      __builtin_amdgcn_s_waitcnt(0x3f70);  // K(0), V(0), K(1) and the Q rows have landed
      if (lag) asm volatile("s_barrier" ::: "memory");
      asm volatile("s_barrier" ::: "memory");
#pragma unroll 1
      for (int i = 0; i < n; ++i) {
        const bool act = active(i);
        // ---- S^T = K Q^T (K of tile i landed before the previous second barrier) ----
        f32x16 acc_s[NB];
        if (act) {
          const uint8_t* kb = kbuf(i);
          constexpr int NJ = NB * NKK;
          auto rd = [&](int j) {
            return *reinterpret_cast<const u32x4*>(kb + koff[j % NKK] + 32 * (j / NKK) * ROWB);
          };
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc_s[nb] = f32x16{};
          u32x4 fa[4];
          fa[0] = rd(0);
          fa[1] = rd(1);
          fa[2] = rd(2);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            if (j + 3 < NJ) fa[(j + 3) % 4] = rd(j + 3);
            const int kk = j % NKK;
            const u32x4 bq = {qf[4 * kk], qf[4 * kk + 1], qf[4 * kk + 2], qf[4 * kk + 3]};
            acc_s[j / NKK] = Tag::mfma32(fa[j % 4], bq, acc_s[j / NKK]);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 1);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            if (j + 3 < NJ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
          }
        }
        // first barrier: sets the phase of the two halves
        asm volatile("s_barrier" ::: "memory");
        // ---- mask, lazy online softmax ----
        uint32_t pf[CPB][4];
        if (act) {
          const int key0 = (t0 + HALVES * i + half) * BN;
          if ((key0 + BN > Skv) || (CAUSAL && key0 + BN - 1 > qoff + pw0)) {
            asm volatile("" ::: "memory");
            const int lim = (CAUSAL ? min(qoff + qpos, Skv - 1) : Skv - 1) - key0 - 4 * hh;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (32 * nb + 8 * (r >> 2) + (r & 3) > lim) acc_s[nb][r] = kNegInf;
          }
          float mx = kNegInf;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc_s[nb][r]);
          mx = pair_max32(mx) * p.scale_log2;
          if (__ballot(mx > m_ref + kLazy)) {
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_ref - m_new);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
            m_ref = m_new;
          }
          const float m_use = m_ref == kNegInf ? 0.f : m_ref;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              const float e0 = fast_exp2(fmaf(acc_s[nb][r], p.scale_log2, -m_use));
              const float e1 = fast_exp2(fmaf(acc_s[nb][r + 1], p.scale_log2, -m_use));
              const uint32_t pk = Tag::pack2(e0, e1);
              pf[2 * nb + (r >> 3)][(r & 7) >> 1] = pk;
              l_run = Tag::sum2(pk, l_run);
            }
        }
        // second barrier: V(i) and K(i+1) of every wave of this half have
        // landed, and every wave of the half is done with V(i-1) and K(i)
        __builtin_amdgcn_s_waitcnt(0x3f70);
        asm volatile("s_barrier" ::: "memory");
        // ---- O^T += V^T P^T ----
        if (act) {
          const uint8_t* vb = vbuf(i);
          constexpr int NJ = NDB * CPB;
          auto rd = [&](int j) {
            const int db = j / CPB, c = j % CPB;
            const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(v4i16, vb + voff[db] + 16 * c * ROWB));
            const v4i16 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(v4i16, vb + voff[db] + (16 * c + 8) * ROWB));
            const u32x2 a1 = __builtin_bit_cast(u32x2, x1), a2 = __builtin_bit_cast(u32x2, x2);
            return u32x4{a1[0], a1[1], a2[0], a2[1]};
          };
          u32x4 fa[3];
          fa[0] = rd(0);
          fa[1] = rd(1);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            if (j + 2 < NJ) fa[(j + 2) % 3] = rd(j + 2);
            const int c = j % CPB;
            const u32x4 bp = {pf[c][0], pf[c][1], pf[c][2], pf[c][3]};
            acc_o[j / CPB] = Tag::mfma32(fa[j % 3], bp, acc_o[j / CPB]);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (j + 2 < NJ) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
        }
        // V(i+1) and K(i+2) into the stages of V(i-1) and K(i).  Issued after
        // the transposing reads of V(i): the compiler makes those reads wait
        // for every LDS DMA in flight, so loads issued before them would
        // stall the PV MFMAs until they land.
        if (exists(i + 1)) dma(vg, vbuf(i + 1), dv, i + 1);
        if (exists(i + 2)) dma(kg, kbuf(i + 2), dk, i + 2);
      }
      if (!lag) asm volatile("s_barrier" ::: "memory");
    } else {
#pragma unroll 1
    for (int i = 0; i < n; ++i) {
      __builtin_amdgcn_s_waitcnt(0x3f70);  // this thread's loads of tile i have landed
      __syncthreads();                     // ... and everybody's; stage (i+1)&1 is free
      const bool has_next = exists(i + 1);
      if (has_next) {
        if (RS) {
          stage_load(i + 1);
        } else {
          dma(vg, vbuf(i + 1), dv, i + 1);
          if (RK) load_k_regs(i + 1);
          else dma(kg, kbuf(i + 1), dk, i + 1);
        }
      }
      if (RK) rope_base_fill(i + 2);

      if (active(i)) {
        // ---- S^T = K Q^T; A operands read from LDS three MFMAs ahead ----
        f32x16 acc_s[NB];
        {
          const uint8_t* kb = kbuf(i);
          constexpr int NJ = NB * NKK;  // MFMA j = NKK nb + kk
          auto rd = [&](int j) {
            return *reinterpret_cast<const u32x4*>(kb + koff[j % NKK] + 32 * (j / NKK) * ROWB);
          };
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc_s[nb] = f32x16{};
          u32x4 fa[4];
          fa[0] = rd(0);
          fa[1] = rd(1);
          fa[2] = rd(2);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            if (j + 3 < NJ) fa[(j + 3) % 4] = rd(j + 3);
            const int kk = j % NKK;
            const u32x4 bq = {qf[4 * kk], qf[4 * kk + 1], qf[4 * kk + 2], qf[4 * kk + 3]};
            acc_s[j / NKK] = Tag::mfma32(fa[j % 4], bq, acc_s[j / NKK]);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 1);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            if (j + 3 < NJ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
          }
        }
        // ---- mask, lazy online softmax ----
        // only tiles that cross the diagonal or the end of the sequence are
        // masked; the empty asm keeps this a branch (not per-element selects)
        const int key0 = (t0 + HALVES * i + half) * BN;
        if ((key0 + BN > Skv) || (CAUSAL && key0 + BN - 1 > qoff + pw0)) {
          asm volatile("" ::: "memory");
          // key = key0 + 4 hh + off(nb, r) is visible iff key <= min(qpos, S - 1)
          const int lim = (CAUSAL ? min(qoff + qpos, Skv - 1) : Skv - 1) - key0 - 4 * hh;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * nb + 8 * (r >> 2) + (r & 3) > lim) acc_s[nb][r] = kNegInf;
        }
        float mx = kNegInf;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc_s[nb][r]);
        mx = pair_max32(mx) * p.scale_log2;
        if (__ballot(mx > m_ref + kLazy)) {
          const float m_new = fmaxf(m_ref, mx);
          // 0 when m_ref = -inf; 1 for a row that has seen no key yet (both -inf)
          const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_ref - m_new);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
          m_ref = m_new;
        }
        const float m_use = m_ref == kNegInf ? 0.f : m_ref;
        uint32_t pf[CPB][4];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float e0 = fast_exp2(fmaf(acc_s[nb][r], p.scale_log2, -m_use));
            const float e1 = fast_exp2(fmaf(acc_s[nb][r + 1], p.scale_log2, -m_use));
            const uint32_t pk = Tag::pack2(e0, e1);
            pf[2 * nb + (r >> 3)][(r & 7) >> 1] = pk;
            l_run = Tag::sum2(pk, l_run);  // row sum of the rounded probabilities
          }
        // ---- O^T += V^T P^T; transposing reads issued two MFMAs ahead ----
        {
          const uint8_t* vb = vbuf(i);
          constexpr int NJ = NDB * CPB;  // MFMA j = CPB db + c
          auto rd = [&](int j) {
            const int db = j / CPB, c = j % CPB;
            const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(v4i16, vb + voff[db] + 16 * c * ROWB));
            const v4i16 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(v4i16, vb + voff[db] + (16 * c + 8) * ROWB));
            const u32x2 a1 = __builtin_bit_cast(u32x2, x1), a2 = __builtin_bit_cast(u32x2, x2);
            return u32x4{a1[0], a1[1], a2[0], a2[1]};
          };
          u32x4 fa[3];
          fa[0] = rd(0);
          fa[1] = rd(1);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            if (j + 2 < NJ) fa[(j + 2) % 3] = rd(j + 2);
            const int c = j % CPB;
            const u32x4 bp = {pf[c][0], pf[c][1], pf[c][2], pf[c][3]};
            acc_o[j / CPB] = Tag::mfma32(fa[j % 3], bp, acc_o[j / CPB]);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (j + 2 < NJ) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
        }
      }
      if (RK && has_next) rotate_store_k(i + 1);
      if (RS && has_next) stage_store(i + 1);  // stage (i+1)&1: tile i-1, done by every wave
    }
    }  // PP

    // ---- merge the two halves (same rows, disjoint key tiles) ----
    float* sc = reinterpret_cast<float*>(smem) + wq * (NDB * 16 + 2) * 64;
    if (HALVES == 2) __syncthreads();
    if (HALVES == 2 && half == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[(db * 16 + r) * 64 + lane] = acc_o[db][r];
      sc[(NDB * 16) * 64 + lane] = m_ref;
      sc[(NDB * 16 + 1) * 64 + lane] = l_run;
    }
    if (HALVES == 2) __syncthreads();
    if (half == 0) {
      const float m1 = HALVES == 2 ? sc[(NDB * 16) * 64 + lane] : kNegInf;
      const float l1 = HALVES == 2 ? sc[(NDB * 16 + 1) * 64 + lane] : 0.f;
      const float M = fmaxf(m_ref, m1);
      const float Mu = M == kNegInf ? 0.f : M;
      const float f0 = fast_exp2(m_ref - Mu), f1 = fast_exp2(m1 - Mu);
      const float l = pair_sum32(l_run * f0 + l1 * f1);
      const float inv = l > 0.f ? p.out_scale / l : 0.f;
      // chunk mode with several key ranges: this item's result (normalised
      // within its range) and its log-sum-exp go to the split workspace
      // [rows, nsplit, D] / [rows, nsplit] for the combine step
      const bool to_ws = CHUNK && p.nsplit > 1;
      const size_t row = ((size_t)b * p.Hq + head) * p.S + qpos;
      if constexpr (CHUNK) {
        // chunk mode: O (or this key range's part of it) leaves through LDS,
        // so that each store instruction writes 16-byte pieces of whole rows
        // instead of touching 32 rows (a lane's accumulator holds 4-element
        // pieces of one row).  Wave wq transposes through quarter wq of the
        // stage memory once every wave is past its key loop; the item loop's
        // barrier keeps the next item's loads out until all have read back.
        uint8_t* area = smem + wq * TILEB;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        int lm = m, ln = lane;
        asm volatile("" : "+v"(lm), "+v"(ln));  // keep the addresses below out of the item loop
        auto stage_out = [&](auto odt) {
          constexpr int OD = decltype(odt)::value;
          constexpr int ES = OD == ATTN_F32 ? 4 : 2;
          constexpr int RB = D * ES;    // bytes per output row
          constexpr int CPR = RB / 16;  // 16-byte pieces per row (XOR-swizzled by row)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int byte = (32 * db + 8 * g4 + 4 * hh) * ES;
              uint8_t* dst = area + lm * RB + 16 * ((byte / 16) ^ (lm % CPR)) + byte % 16;
              const float o0 = acc_o[db][4 * g4] * inv, o1 = acc_o[db][4 * g4 + 1] * inv;
              const float o2 = acc_o[db][4 * g4 + 2] * inv, o3 = acc_o[db][4 * g4 + 3] * inv;
              if constexpr (OD == ATTN_F32) *reinterpret_cast<f32x4*>(dst) = f32x4{o0, o1, o2, o3};
              else if constexpr (OD == ATTN_BF16) *reinterpret_cast<u32x2*>(dst) = u32x2{Bf16Tag::pack2(o0, o1), Bf16Tag::pack2(o2, o3)};
              else *reinterpret_cast<u32x2*>(dst) = u32x2{F16Tag::pack2(o0, o1), F16Tag::pack2(o2, o3)};
            }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's LDS writes are done before its reads
          constexpr int RPR = 64 / CPR;  // rows per read instruction
          // destination row r of this wave: query row pw0 + r; parts of
          // consecutive rows are nsplit pieces apart in the split workspace
          const size_t rstride = (size_t)(to_ws ? p.nsplit : 1) * RB;
          uint8_t* obase = reinterpret_cast<uint8_t*>(to_ws ? static_cast<void*>(p.ws_o) : p.o) +
                           ((((size_t)b * p.Hq + head) * p.S + pw0) * (to_ws ? p.nsplit : 1) + (to_ws ? split : 0)) * RB;
          u32x4 ov[32 / RPR];
#pragma unroll
          for (int i = 0; i < 32 / RPR; ++i) {
            const int r = RPR * i + ln / CPR, c = ln % CPR;
            ov[i] = *reinterpret_cast<const u32x4*>(area + r * RB + 16 * (c ^ (r % CPR)));
          }
          // stores at device scope (sc1) through a buffer whose range ends
          // after this wave's last row in the chunk (rows past it, or a wave
          // with none, are dropped): measured 952 -> 933 us on the chunked
          // 2048-token prompt against plain stores, 961 with non-temporal sc1
          const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
              obase, (short)0, (int)(max(0, min(p.S - pw0, 32)) * rstride), kBufferRsrcWord3);
#pragma unroll
          for (int i = 0; i < 32 / RPR; ++i) {
            const int r = RPR * i + ln / CPR, c = ln % CPR;
            __builtin_amdgcn_raw_buffer_store_b128(ov[i], ors, (int)(r * rstride) + 16 * c, 0, ATTN_CHUNK_OAUX);
          }
        };
        if (to_ws) stage_out(ic_t<ATTN_CHUNK_BF16_PARTS ? ATTN_BF16 : ATTN_F32>{});
        else if (p.out_dtype == ATTN_F32) stage_out(ic_t<ATTN_F32>{});
        else if (p.out_dtype == ATTN_BF16) stage_out(ic_t<ATTN_BF16>{});
        else stage_out(ic_t<ATTN_F16>{});
        if (qpos < p.S && hh == 0) {
          const float lse_row = l > 0.f ? (Mu + __log2f(l)) * kLn2 : kNegInf;
          if (to_ws) p.ws_lse[row * p.nsplit + split] = lse_row;
          else if (p.lse) p.lse[row] = lse_row;
        }
      } else if (qpos < p.S) {
        const size_t obase = to_ws ? (row * p.nsplit + split) * D : row * D;
        void* const obuf = to_ws ? static_cast<void*>(p.ws_o) : p.o;
        const int odt = to_ws ? (int)ATTN_F32 : p.out_dtype;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float v4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * g4 + e;
              v4[e] = (HALVES == 2 ? acc_o[db][r] * f0 + sc[(db * 16 + r) * 64 + lane] * f1 : acc_o[db][r]) * inv;
            }
            store4(obuf, obase + 32 * db + 8 * g4 + 4 * hh, odt, v4[0], v4[1], v4[2], v4[3]);
          }
        const float lse_row = l > 0.f ? (Mu + __log2f(l)) * kLn2 : kNegInf;
        if (to_ws && hh == 0) p.ws_lse[row * p.nsplit + split] = lse_row;
        else if (p.lse && hh == 0) p.lse[row] = lse_row;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined MFMA kernel.  Same work split and LDS layout as
// prefill_fwd_kernel with 4-wave workgroups (32 query rows per wave, 64-key
// tiles), but the key loop is skewed by one tile: while a wave exponentiates
// the scores of tile i it already issues the S = K Q^T MFMAs of tile i+1, so
// the matrix cores stay busy through the softmax instead of waiting for it.
// K is therefore staged one tile ahead of V.  With RoPE the raw K tile is
// DMA'd to LDS and rotated in place by the wave that loaded its rows.  The
// row max of tile i+1 is taken while the PV MFMAs of tile i run, and the V
// loads of tile i+1 are issued between the two phases instead of in one
// burst after the barrier.  On gfx950 this measures about equal to the
// unskewed kernel (ahead only at long sequences): it is a sweep
// configuration, not the default.
// ---------------------------------------------------------------------------
template <class Tag, int D, bool CAUSAL, int ROPE>
__global__ __launch_bounds__(256, 2) void prefill_pipe_kernel(const PrefillParams p) {
  // RoPE mode: 0 none; 1 Q and K rotated here; 2 Q rotated here, K already
  // rotated in HBM
  constexpr bool RQ = ROPE != 0, RK = ROPE == 1;
  constexpr int BN = 64;
  constexpr int ROWB = D * 2;        // bytes per K/V row
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int TILEB = BN * ROWB;   // bytes of one K or V tile
  constexpr int RPI = 64 / CH;       // rows per wave-wide direct load
  constexpr int IPW = BN / RPI / 4;  // direct loads per wave per tile
  constexpr int NKK = D / 16, NDB = D / 32, HALF = D / 2, PAIRS = D / 64;
  constexpr float kLazy = 8.f;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILEB];  // [K0 K1 V0 V1]
  __shared__ float rope_base[2][RK ? D : 1];                        // [slot][cos | sin]

  // chunk swizzles (see prefill_fwd_kernel)
  auto kswz = [](int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); };
  auto vswz = [](int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wq = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int m = lane & 31, hh = lane >> 5;
  const int g = lane >> 4, rr = lane & 15;

  int koff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) koff[kk] = m * ROWB + 16 * ((2 * kk + hh) ^ kswz(m));
  int voff[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d = 32 * db + 16 * (g & 1) + 4 * (rr & 3);
    const int key = 4 * (g >> 1) + (rr >> 2);
    voff[db] = key * ROWB + 16 * ((d >> 3) ^ vswz(key)) + 2 * (d & 7);
  }
  // direct-load lane offsets for the first of the wave's IPW loads; wave wq
  // loads rows 16 wq .. 16 wq + 15 of a tile, RPI rows per load.  Load u
  // reads RPI u rows further on and, since the V swizzle does not depend on
  // the row bits that u sets, V load u is load 0 moved by u RPI ROWB bytes
  // (an instruction offset, applied to both the global and the LDS
  // address).  The K swizzle XORs 4 u into the chunk index of those rows,
  // so K load u also XORs 64 u into the byte offset (no carry: the row part
  // of the offset is a multiple of 128 and the chunk part stays below it).
  const int row0 = RPI * wq * IPW + lane / CH, phys0 = lane % CH;
  const int dk0 = row0 * ROWB + 16 * (phys0 ^ kswz(row0));
  const int dv0 = row0 * ROWB + 16 * (phys0 ^ vswz(row0));

  // causal: the second half of the grid takes the short items in reverse
  // order so that workgroups k and k + n/2 carry complementary work
  const int per_ptile = p.B * p.Hkv * p.n_hgroups;
  const int n_items = p.n_ptiles * per_ptile;
  const int half_items = (n_items + 1) / 2;
  const int item = (CAUSAL && (int)blockIdx.x >= half_items) ? n_items - 1 - ((int)blockIdx.x - half_items)
                                                             : (int)blockIdx.x;
  // RoPE on K: this thread rotates row kr (one of the rows its own wave
  // loaded) at chunk pairs (kj + 4u, + CH/2)
  const int kr = (lane & 15) + 16 * wq, kj = lane >> 4;
  const float fhi_lane = RK && lane < HALF ? p.rope_fhi[lane] : 0.f;
  const float flo_lane = RK && lane < HALF ? p.rope_flo[lane] : 0.f;
  float rcos[RK ? 8 * PAIRS : 1], rsin[RK ? 8 * PAIRS : 1];
  if (RK) {
#pragma unroll
    for (int u = 0; u < PAIRS; ++u)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int j = 8 * (kj + 4 * u) + t;
        const float rev = __builtin_amdgcn_fractf((float)(kr & 63) * p.rope_fhi[j]) + (float)(kr & 63) * p.rope_flo[j];
        rcos[8 * u + t] = __builtin_amdgcn_cosf(rev);
        rsin[8 * u + t] = __builtin_amdgcn_sinf(rev);
      }
  }

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
  const int n = (kend + BN - 1) / BN;
  const int qpos = pw0 + m;

  // ---- Q fragments (B operand of S^T = K Q^T), rotated in registers ----
  uint32_t qf[D / 4];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + (((size_t)b * p.Hq + head) * p.S + qpos) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 w = qpos < p.S ? ldg16(qrow + 16 * kk + 8 * hh) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * kk + e] = w[e];
    }
    if (RQ) {
#pragma unroll
      for (int kk = 0; kk < NKK / 2; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w1 = qf[4 * kk + e], w2 = qf[4 * (kk + NKK / 2) + e];
          float r1[2], r2[2];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int fi = 16 * kk + 8 * hh + 2 * e + s;
            const float rev = __builtin_amdgcn_fractf((float)qpos * p.rope_fhi[fi]) + (float)qpos * p.rope_flo[fi];
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
  auto exists = [&](int i) { return i < n; };
  auto kbuf = [&](int i) { return smem + (i & 1) * TILEB; };
  auto vbuf = [&](int i) { return smem + (2 + (i & 1)) * TILEB; };

  // direct HBM -> LDS load of tile i of K or V; rows past S read as zero
  auto dma = [&](const uint8_t* src, uint8_t* dst, bool is_k, int i) {
    const int key0 = i * BN;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(src + (size_t)key0 * ROWB), (short)0, (p.S - key0) * ROWB, kBufferRsrcWord3);
    auto* ld = LDS_AS(void, dst + RPI * wq * IPW * ROWB);
    // (the instruction offset must be a constant: loads written out)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, ld, 16, is_k ? dk0 : dv0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, ld, 16, is_k ? (dk0 ^ 64) : dv0, 0, RPI * ROWB, 0);
    if constexpr (IPW == 4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, ld, 16, is_k ? (dk0 ^ 128) : dv0, 0, 2 * RPI * ROWB, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, ld, 16, is_k ? (dk0 ^ 192) : dv0, 0, 3 * RPI * ROWB, 0);
    }
  };
  // cos / sin of the base angle key0 f_j of tile i into table slot i & 1
  auto rope_base_fill = [&](int i) {
    if (wq == 0 && lane < HALF) {
      const float key0 = (float)(i * BN);
      const float rev = __builtin_amdgcn_fractf(key0 * fhi_lane) + key0 * flo_lane;
      rope_base[i & 1][lane] = __builtin_amdgcn_cosf(rev);
      rope_base[i & 1][HALF + lane] = __builtin_amdgcn_sinf(rev);
    }
  };
  // rotate this thread's pairs of K tile i in place (angle addition of the
  // tile base angle and the row offset angle)
  auto rotate_k = [&](int i) {
    uint8_t* kb = kbuf(i);
#pragma unroll
    for (int u = 0; u < PAIRS; ++u) {
      const int c = kj + 4 * u;
      u32x4* plo = reinterpret_cast<u32x4*>(kb + kr * ROWB + 16 * (c ^ kswz(kr)));
      u32x4* phi = reinterpret_cast<u32x4*>(kb + kr * ROWB + 16 * ((c + CH / 2) ^ kswz(kr)));
      u32x4 lo = *plo, hi = *phi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float r1[2], r2[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int j = 8 * c + 2 * e + s, t = 8 * u + 2 * e + s;
          const float cb = rope_base[i & 1][j], sb = rope_base[i & 1][HALF + j];
          const float cs = cb * rcos[t] - sb * rsin[t], sn = sb * rcos[t] + cb * rsin[t];
          const float x1 = Tag::to_f32(s ? (lo[e] >> 16) : (lo[e] & 0xffff));
          const float x2 = Tag::to_f32(s ? (hi[e] >> 16) : (hi[e] & 0xffff));
          r1[s] = x1 * cs - x2 * sn;
          r2[s] = x2 * cs + x1 * sn;
        }
        lo[e] = Tag::pack2(r1[0], r1[1]);
        hi[e] = Tag::pack2(r2[0], r2[1]);
      }
      *plo = lo;
      *phi = hi;
    }
  };

  // ---- running state ----
  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_ref = kNegInf;  // exponent reference (scaled log2 domain), equal in both lanes of a row
  float l_run = 0.f;      // sum over this lane's keys of exp2(s - m_ref)

  // S^T of tile i into acc (MFMA j: k-step j / 2, key block j % 2); K
  // fragments read from LDS three MFMAs ahead
  auto k_frag = [&](const uint8_t* kb, int j) {
    return *reinterpret_cast<const u32x4*>(kb + koff[j >> 1] + 32 * (j & 1) * ROWB);
  };
  auto scores = [&](int i, f32x16 (&acc)[2]) {
    const uint8_t* kb = kbuf(i);
    constexpr int NJ = 2 * NKK;
    acc[0] = f32x16{};
    acc[1] = f32x16{};
    u32x4 fa[4];
    fa[0] = k_frag(kb, 0);
    fa[1] = k_frag(kb, 1);
    fa[2] = k_frag(kb, 2);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + 3 < NJ) fa[(j + 3) % 4] = k_frag(kb, j + 3);
      const int kk = j >> 1;
      const u32x4 bq = {qf[4 * kk], qf[4 * kk + 1], qf[4 * kk + 2], qf[4 * kk + 3]};
      acc[j & 1] = Tag::mfma32(fa[j % 4], bq, acc[j & 1]);
    }
  };
  // probabilities of the scores in acc (bf16/f16, B-operand layout of PV)
  // and their row sum
  // (MASK: keys past lim get probability 0)
  auto exponentiate = [&](f32x16 (&acc)[2], float m_use, uint32_t (&pf)[4][4], int lim, auto mask) {
    constexpr bool MASK = decltype(mask)::value;
    auto arg = [&](int nb, int r) {
      const float x = fmaf(acc[nb][r], p.scale_log2, -m_use);
      return (MASK && 32 * nb + 8 * (r >> 2) + (r & 3) > lim) ? kNegInf : x;
    };
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float e0 = fast_exp2(arg(nb, r));
        const float e1 = fast_exp2(arg(nb, r + 1));
        const uint32_t pk = Tag::pack2(e0, e1);
        pf[2 * nb + (r >> 3)][(r & 7) >> 1] = pk;
        l_run = Tag::sum2(pk, l_run);
      }
  };
  // mask, row max and (lazy) rescale for the scores of tile i; returns the
  // exponent offset for exponentiate
  // scaled row max of the scores in acc (both lanes of a row agree); a
  // tree of depth 4 rather than a 16-deep chain
  auto row_max = [&](const f32x16 (&acc)[2], int lim, auto mask) {
    constexpr bool MASK = decltype(mask)::value;
    auto val = [&](int e) {  // element e = 16 nb + r
      const int nb = e >> 4, r = e & 15;
      return (MASK && 32 * nb + 8 * (r >> 2) + (r & 3) > lim) ? kNegInf : acc[nb][r];
    };
    float t1[11];
#pragma unroll
    for (int u = 0; u < 10; ++u) t1[u] = fmaxf(fmaxf(val(3 * u), val(3 * u + 1)), val(3 * u + 2));
    t1[10] = fmaxf(val(30), val(31));
    const float t2a = fmaxf(fmaxf(t1[0], t1[1]), t1[2]), t2b = fmaxf(fmaxf(t1[3], t1[4]), t1[5]);
    const float t2c = fmaxf(fmaxf(t1[6], t1[7]), t1[8]), t2d = fmaxf(t1[9], t1[10]);
    return pair_max32(fmaxf(fmaxf(t2a, t2b), fmaxf(t2c, t2d))) * p.scale_log2;
  };
  // tiles that cross the diagonal or the end of the sequence are masked:
  // key offset o inside the tile (this lane's keys start at 4 hh) is
  // visible iff o <= lim
  auto needs_mask = [&](int i) { return (i * BN + BN > p.S) || (CAUSAL && i * BN + BN - 1 > pw0); };
  auto mask_lim = [&](int i) { return (CAUSAL ? min(qpos, p.S - 1) : p.S - 1) - i * BN - 4 * hh; };
  // (lazy) rescale for the scores of tile i with row max mx (the unmasked
  // max taken while the previous tile's PV ran, or the masked max); returns
  // the exponent offset for exponentiate
  auto softmax_head = [&](float mx) {
    if (__ballot(mx > m_ref + kLazy)) {
      const float m_new = fmaxf(m_ref, mx);
      // 0 when m_ref = -inf; 1 for a row that has seen no key yet (both -inf)
      const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
      m_ref = m_new;
    }
    return m_ref == kNegInf ? 0.f : m_ref;
  };
  // O^T += V^T P^T for tile i; transposing reads issued two MFMAs ahead
  auto pv = [&](int i, const uint32_t (&pf)[4][4], auto own_schedule) {
    const uint8_t* vb = vbuf(i);
    constexpr int NJ = NDB * 4;  // MFMA j = NDB c + db (consecutive MFMAs use different accumulators)
    auto rd = [&](int j) {
      const int db = j % NDB, c = j / NDB;
      const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(v4i16, vb + voff[db] + 16 * c * ROWB));
      const v4i16 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(v4i16, vb + voff[db] + (16 * c + 8) * ROWB));
      const u32x2 a1 = __builtin_bit_cast(u32x2, x1), a2 = __builtin_bit_cast(u32x2, x2);
      return u32x4{a1[0], a1[1], a2[0], a2[1]};
    };
    u32x4 fa[3];
    fa[0] = rd(0);
    fa[1] = rd(1);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + 2 < NJ) fa[(j + 2) % 3] = rd(j + 2);
      const int c = j / NDB;
      const u32x4 bp = {pf[c][0], pf[c][1], pf[c][2], pf[c][3]};
      acc_o[j % NDB] = Tag::mfma32(fa[j % 3], bp, acc_o[j % NDB]);
    }
    if constexpr (decltype(own_schedule)::value) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (j + 2 < NJ) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  };

  // One key tile that has a successor: cur holds S of tile i, nxt receives
  // S of tile i + 1.
  //   top:  tile i's V and tile i+1's K have landed (and K is rotated);
  //         issue V(i+1) and K(i+2) into the stages of tiles i-1 and i
  //   body: softmax of tile i with the MFMAs of S(i+1) interleaved, then PV.
  // A wave whose rows end inside tile i still computes S(i+1) (unused): that
  // keeps the interleaved region one basic block.
  float mx_pre = kNegInf;  // unmasked scaled row max of the next tile's scores
  // the item's last tile, masked (done without a successor to overlap with)
  auto tail_block = [&](int i, f32x16 (&cur)[2]) {
    const int lim = mask_lim(i);
    uint32_t pf[4][4];
    const float m_use = softmax_head(row_max(cur, lim, std::true_type{}));
    exponentiate(cur, m_use, pf, lim, std::true_type{});
    pv(i, pf, std::true_type{});
  };
  // One key tile with a successor: cur holds S of tile i, nxt receives S of
  // tile i + 1.
  //   top:  tile i's V and tile i+1's K have landed (and K is rotated);
  //         issue K(i+2) into the stage tile i used
  //   body: softmax of tile i with the MFMAs of S(i+1) interleaved, then PV
  //         with the loads of V(i+1) and the row max of S(i+1) in between.
  // LAST_TWO: tile i is the item's second to last (no K(i+2) to stage).
  // Every wave does every tile of the item.  Tiles before the last two are
  // never masked.  A wave's diagonal tile is n-1, or n-2 when the four
  // waves hold consecutive 32-row blocks of one head (then the wave's last
  // tile is fully masked, which leaves its running max, sum and output
  // unchanged); the ragged end of the sequence falls in tile n-1.  So the
  // last two tiles are masked and the others are not.
  auto step = [&](int i, f32x16 (&cur)[2], f32x16 (&nxt)[2], auto last_two) {
    __builtin_amdgcn_s_waitcnt(0x3f70);  // this thread's loads have landed
    __syncthreads();                     // ... and everybody's; stages of tiles i-1 / i are free
    if (!decltype(last_two)::value) dma(kg, kbuf(i + 2), true, i + 2);
    if (RK) rope_base_fill(i + 3);
    {
      const int lim = mask_lim(i);
      const float m_use = softmax_head(decltype(last_two)::value ? row_max(cur, lim, last_two) : mx_pre);
      uint32_t pf[4][4];
      scores(i + 1, nxt);
      exponentiate(cur, m_use, pf, lim, last_two);
      dma(vg, vbuf(i + 1), false, i + 1);
      pv(i, pf, std::false_type{});
      mx_pre = row_max(nxt, 0, std::false_type{});
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 1);
#pragma unroll
      for (int j = 0; j < 2 * NKK; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x402, 6, 1);
      }
#pragma unroll
      for (int j = 0; j < 4 * NDB; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        if (j < IPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x402, 2, 1);
      }
    }
    if (RK && !decltype(last_two)::value) {
      __builtin_amdgcn_s_waitcnt(0x3f70);  // raw K(i+2) rows of this wave have landed
      rotate_k(i + 2);
    }
  };
  // the item's last tile
  auto last_step = [&](int i, f32x16 (&cur)[2]) {
    __builtin_amdgcn_s_waitcnt(0x3f70);
    __syncthreads();
    tail_block(i, cur);
  };

  // ---- prologue: K(0), V(0), K(1) staged (and rotated), S(0) computed ----
  f32x16 s_a[2], s_b[2];
  if (RK) {
    rope_base_fill(0);
    rope_base_fill(1);
  }
  dma(kg, kbuf(0), true, 0);
  dma(vg, vbuf(0), false, 0);
  if (exists(1)) dma(kg, kbuf(1), true, 1);
  __builtin_amdgcn_s_waitcnt(0x3f70);
  if (RK) {
    __syncthreads();  // base table visible
    rotate_k(0);
    if (exists(1)) rotate_k(1);
    __syncthreads();  // rotated tiles visible; table slot 0 free
    rope_base_fill(2);
  }
  __syncthreads();
  scores(0, s_a);
  mx_pre = row_max(s_a, 0, std::false_type{});

  // Tiles 0 .. n-3 have an active successor for every wave (a wave's rows
  // end in tile n-2 or n-1), so the loop takes no tail; the last two tiles
  // follow it (after moving the scores to s_a when the loop count is odd).
  int i = 0;
#pragma unroll 1
  for (; i + 3 < n; i += 2) {
    step(i, s_a, s_b, std::false_type{});
    step(i + 1, s_b, s_a, std::false_type{});
  }
  if (n - i == 3) {
    step(i, s_a, s_b, std::false_type{});
    ++i;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) s_a[nb] = s_b[nb];
  }
  if (n - i == 2) {
    step(i, s_a, s_b, std::true_type{});
    last_step(i + 1, s_b);
  } else {
    last_step(i, s_a);
  }

  // ---- epilogue ----
  const float Mu = m_ref == kNegInf ? 0.f : m_ref;
  const float l = pair_sum32(l_run);
  const float inv = l > 0.f ? p.out_scale / l : 0.f;
  if (qpos < p.S) {
    const size_t obase = (((size_t)b * p.Hq + head) * p.S + qpos) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int r = 4 * g4;
        store4(p.o, obase + 32 * db + 8 * g4 + 4 * hh, p.out_dtype, acc_o[db][r] * inv, acc_o[db][r + 1] * inv,
               acc_o[db][r + 2] * inv, acc_o[db][r + 3] * inv);
      }
    if (p.lse && hh == 0)
      p.lse[((size_t)b * p.Hq + head) * p.S + qpos] = l > 0.f ? (Mu + __log2f(l)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// fp32 SIMT kernel: L = 8 lanes per query row, 64 rows per workgroup.  Lane
// g of a row holds the rotate-half pairs (i, i + D/2) for i in
// [g D/(2L), (g+1) D/(2L)), so RoPE on Q stays inside the lane; the partial
// dot products of the L lanes are summed with xor shuffles and every lane
// runs the same online softmax over its share of the output.
// ---------------------------------------------------------------------------
// cos / sin of angle pos * w_i for the fp32 kernel: the angle is reduced to
// one revolution exactly (three-part frequency split) before the radian
// conversion, so its error does not grow with the position.
__device__ inline void rope_sincos_exact(const PrefillParams& p, int pos, int i, float* sn, float* cs) {
  const float fp = (float)pos;
  const float rev = __builtin_amdgcn_fractf(__builtin_amdgcn_fractf(fp * p.rope_fhi[i]) +
                                            __builtin_amdgcn_fractf(fp * p.rope_fmid[i]) + fp * p.rope_flo[i]);
  sincosf(6.283185307179586f * rev, sn, cs);
}

constexpr int kF32Lanes = 8;  // lanes per query row of the fp32 kernel

template <int D, bool CAUSAL, bool ROPE>
__global__ __launch_bounds__(64 * kF32Lanes) void prefill_f32_kernel(const PrefillParams p) {
  constexpr int BN = 32;
  constexpr int HALF = D / 2;
  constexpr int LPR = kF32Lanes;    // lanes per query row
  constexpr int NT = 64 * LPR;      // threads per workgroup (64 rows)
  constexpr int QP = HALF / LPR;    // rotate-half pairs per lane
  __shared__ float ks[BN][D];
  __shared__ float vs[BN][D];
  const int tid = threadIdx.x;
  const int g = tid & (LPR - 1), rl = tid / LPR;  // lane of the row, row of the workgroup
  const int head = blockIdx.y, b = blockIdx.z;
  const int kvh = head / p.G;
  const int r0 = blockIdx.x * 64;
  const int qpos = r0 + rl;
  const int i0 = g * QP;  // this lane's pairs: dims i0 .. i0+QP-1 and HALF+i0 ..
  const float* qsrc = reinterpret_cast<const float*>(p.q) + (((size_t)b * p.Hq + head) * p.S + min(qpos, p.S - 1)) * D;
  float q[2 * QP], o[2 * QP];
#pragma unroll
  for (int i = 0; i < QP; ++i) {
    q[i] = qsrc[i0 + i];
    q[QP + i] = qsrc[HALF + i0 + i];
    o[i] = 0.f;
    o[QP + i] = 0.f;
  }
  if (ROPE) {
#pragma unroll
    for (int i = 0; i < QP; ++i) {
      float sn, cs;
      rope_sincos_exact(p, qpos, i0 + i, &sn, &cs);
      const float x1 = q[i], x2 = q[QP + i];
      q[i] = x1 * cs - x2 * sn;
      q[QP + i] = x2 * cs + x1 * sn;
    }
  }
  const int kend = CAUSAL ? min(p.S, r0 + 64) : p.S;
  const float* kbase = reinterpret_cast<const float*>(p.k) + ((size_t)b * p.Hkv + kvh) * p.S * D;
  const float* vbase = reinterpret_cast<const float*>(p.v) + ((size_t)b * p.Hkv + kvh) * p.S * D;
  float m_run = kNegInf, l_run = 0.f;
  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    for (int e = tid; e < BN * D; e += NT) {
      const int r = e / D, d = e % D;
      const int key = k0 + r;
      ks[r][d] = key < p.S ? kbase[(size_t)key * D + d] : 0.f;
      vs[r][d] = key < p.S ? vbase[(size_t)key * D + d] : 0.f;
    }
    if (ROPE) {
      __syncthreads();
      for (int e = tid; e < BN * HALF; e += NT) {
        const int r = e / HALF, i = e % HALF;
        float sn, cs;
        rope_sincos_exact(p, k0 + r, i, &sn, &cs);
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
      for (int i = 0; i < QP; ++i) {
        acc = fmaf(q[i], ks[j][i0 + i], acc);
        acc = fmaf(q[QP + i], ks[j][HALF + i0 + i], acc);
      }
#pragma unroll
      for (int x = 1; x < LPR; x <<= 1) acc += __shfl_xor(acc, x);
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
    for (int i = 0; i < 2 * QP; ++i) o[i] *= alpha;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const float pj = exp2f(s[j] - m_use);
      l_run += pj;
#pragma unroll
      for (int i = 0; i < QP; ++i) {
        o[i] = fmaf(pj, vs[j][i0 + i], o[i]);
        o[QP + i] = fmaf(pj, vs[j][HALF + i0 + i], o[QP + i]);
      }
    }
  }
  if (qpos < p.S) {
    const float inv = l_run > 0.f ? p.out_scale / l_run : 0.f;
    const size_t obase = (((size_t)b * p.Hq + head) * p.S + qpos) * D;
#pragma unroll
    for (int i = 0; i < QP; i += 4) {
      store4(p.o, obase + i0 + i, p.out_dtype, o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv);
      store4(p.o, obase + HALF + i0 + i, p.out_dtype, o[QP + i] * inv, o[QP + i + 1] * inv, o[QP + i + 2] * inv,
             o[QP + i + 3] * inv);
    }
    if (p.lse && g == 0) p.lse[((size_t)b * p.Hq + head) * p.S + qpos] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Host dispatch
// ---------------------------------------------------------------------------
// rope: RoPE mode of the kernels (0 none, 1 Q and K rotated in the kernel,
// 2 Q rotated in the kernel and K already rotated in HBM)
template <class Tag, int D, int H, bool CAUSAL, int RM>
static void launch_fwd_hr(const PrefillParams& p, hipStream_t st) {
  const long long items = (long long)p.n_ptiles * p.B * p.Hkv * p.n_hgroups;
  long long wgs = CAUSAL && H == 2 ? (items + 1) / 2 : items;
  if (H == 1 && p.persist) {
    // two resident workgroups per compute unit loop over the items once
    // there are more than two rounds of them; up to two rounds the hardware
    // dispatcher's refill (one workgroup per item) is as good or better
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    const long long resident = 2LL * (cus > 0 ? cus : 256);
    if (items > 2 * resident) {
      hipLaunchKernelGGL((prefill_fwd_kernel<Tag, D, CAUSAL, RM, 1, false, true>), dim3((unsigned)resident), dim3(256), 0,
                         st, p);
      return;
    }
  }
  if constexpr (H == 1 && RM != 1) {
    if (p.regstage) {
      hipLaunchKernelGGL((prefill_fwd_kernel<Tag, D, CAUSAL, RM, 1, false, false, 64, false, true>),
                         dim3((unsigned)wgs), dim3(256), 0, st, p);
      return;
    }
  }
  if constexpr (H == 2 && RM != 1) {
    if (p.pingpong) {
      hipLaunchKernelGGL((prefill_fwd_kernel<Tag, D, CAUSAL, RM, 2, false, false, 64, true>), dim3((unsigned)wgs),
                         dim3(512), 0, st, p);
      return;
    }
  }
  hipLaunchKernelGGL((prefill_fwd_kernel<Tag, D, CAUSAL, RM, H>), dim3((unsigned)wgs), dim3(256 * H), 0, st, p);
}

template <class Tag, int D, int H>
static void launch_fwd_h(const PrefillParams& p, bool causal, int rope, hipStream_t st) {
  if (causal) {
    if (rope == 1) launch_fwd_hr<Tag, D, H, true, 1>(p, st);
    else if (rope == 2) launch_fwd_hr<Tag, D, H, true, 2>(p, st);
    else launch_fwd_hr<Tag, D, H, true, 0>(p, st);
  } else {
    if (rope == 1) launch_fwd_hr<Tag, D, H, false, 1>(p, st);
    else if (rope == 2) launch_fwd_hr<Tag, D, H, false, 2>(p, st);
    else launch_fwd_hr<Tag, D, H, false, 0>(p, st);
  }
}

template <class Tag, int D>
static void launch_fwd(const PrefillParams& p, bool causal, int rope, hipStream_t st) {
  if (p.halves == 1) launch_fwd_h<Tag, D, 1>(p, causal, rope, st);
  else launch_fwd_h<Tag, D, 2>(p, causal, rope, st);
}

template <class Tag, int D>
static void launch_pipe(const PrefillParams& p, bool causal, int rope, hipStream_t st) {
  const dim3 grid((unsigned)((long long)p.n_ptiles * p.B * p.Hkv * p.n_hgroups)), block(256);
  if (causal) {
    if (rope == 1) hipLaunchKernelGGL((prefill_pipe_kernel<Tag, D, true, 1>), grid, block, 0, st, p);
    else if (rope == 2) hipLaunchKernelGGL((prefill_pipe_kernel<Tag, D, true, 2>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((prefill_pipe_kernel<Tag, D, true, 0>), grid, block, 0, st, p);
  } else {
    if (rope == 1) hipLaunchKernelGGL((prefill_pipe_kernel<Tag, D, false, 1>), grid, block, 0, st, p);
    else if (rope == 2) hipLaunchKernelGGL((prefill_pipe_kernel<Tag, D, false, 2>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((prefill_pipe_kernel<Tag, D, false, 0>), grid, block, 0, st, p);
  }
}

// configuration 4: the 4-wave kernel with 32-key tiles (three workgroups per
// compute unit); RoPE with K rotated per staged tile has no such variant and
// runs as configuration 0
template <class Tag, int D>
static void launch_bn32(const PrefillParams& p, bool causal, int rope, hipStream_t st) {
  const dim3 grid((unsigned)((long long)p.n_ptiles * p.B * p.Hkv * p.n_hgroups)), block(256);
  if (causal) {
    if (rope == 2) hipLaunchKernelGGL((prefill_fwd_kernel<Tag, D, true, 2, 1, false, false, 32>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((prefill_fwd_kernel<Tag, D, true, 0, 1, false, false, 32>), grid, block, 0, st, p);
  } else {
    if (rope == 2) hipLaunchKernelGGL((prefill_fwd_kernel<Tag, D, false, 2, 1, false, false, 32>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((prefill_fwd_kernel<Tag, D, false, 0, 1, false, false, 32>), grid, block, 0, st, p);
  }
}

template <class Tag, int D>
static void launch_16bit(const PrefillParams& p, int config, bool causal, int rope, hipStream_t st) {
  if (config == 2) launch_pipe<Tag, D>(p, causal, rope, st);
  else if (config == 4 && rope != 1) launch_bn32<Tag, D>(p, causal, rope, st);
  else launch_fwd<Tag, D>(p, causal, rope, st);  // 0, 1, 3 (persistent 4-wave)
}

template <class Tag, int D, bool FP8, bool P8 = false>
static void launch_mfma(const PrefillParams& p, bool causal, dim3 grid, hipStream_t st) {
  if (causal) hipLaunchKernelGGL((prefill_mfma_kernel<Tag, D, true, false, FP8, P8>), grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL((prefill_mfma_kernel<Tag, D, false, false, FP8, P8>), grid, dim3(256), 0, st, p);
}

template <int D>
static void launch_f32(const PrefillParams& p, bool causal, bool rope, hipStream_t st) {
  dim3 grid((p.S + 63) / 64, p.Hq, p.B), block(64 * kF32Lanes);  // 64 rows x kF32Lanes lanes
  if (causal) {
    if (rope) hipLaunchKernelGGL((prefill_f32_kernel<D, true, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((prefill_f32_kernel<D, true, false>), grid, block, 0, st, p);
  } else {
    if (rope) hipLaunchKernelGGL((prefill_f32_kernel<D, false, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((prefill_f32_kernel<D, false, false>), grid, block, 0, st, p);
  }
}

}  // namespace attn

using namespace attn;

static attn_status prefill_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int Hq, int Hkv, int S, int D, attn_dtype in_dtype,
                                attn_dtype out_dtype, float softmax_scale, int causal,
                                float rope_theta, float q_descale, float k_descale,
                                float v_descale, int config, void* workspace,
                                size_t workspace_bytes, bool use_ws, hipStream_t stream,
                                bool k_rotated = false) {
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
  p.D = D;
  p.G = Hq / Hkv;
  p.scale_log2 = softmax_scale * q_descale * k_descale * kLog2e;
  p.out_scale = v_descale;
  p.out_dtype = out_dtype;
  p.rope = rope ? 1 : 0;
  p.halves = config == 1 || config == 5 ? 2 : 1;
  p.persist = config == 3 ? 1 : 0;
  p.pingpong = config == 5 ? 1 : 0;
  p.regstage = config == 6 ? 1 : 0;
  if (rope && S > 65536) return ATTN_ERR_UNSUPPORTED;  // exact angle reduction needs pos < 2^16
  if (rope) {
    if (in_dtype == ATTN_F32) attn_host::rope_freq_split(rope_theta, D, p.inv_freq, p.rope_fhi, p.rope_flo, p.rope_fmid);
    else attn_host::rope_freq_split(rope_theta, D, p.inv_freq, p.rope_fhi, p.rope_flo);
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
  // RoPE on K with a workspace: every key is rotated once into the workspace
  // (a K tile is shared by all query tiles of its KV head, so rotating it
  // while staging repeats the work once per query tile); the attention
  // kernel then rotates only its Q rows
  // (k_rotated: the workspace already holds this K rotated; the pre-pass is skipped)
  int rope_mode = rope ? 1 : 0;
  if (rope && use_ws && in_dtype != ATTN_FP8_E5M2) {
    const size_t need = attn_prefill_gqa_rope_workspace_bytes(B, Hkv, S, D, in_dtype, rope_theta);
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!attn_host::aligned(workspace, 16)) return ATTN_ERR_ALIGN;
    if (!k_rotated) {
      const attn_status st = attn_rope_rotate(k, workspace, B, Hkv, S, D, in_dtype, rope_theta, stream);
      if (st != ATTN_OK) return st;
    }
    p.k = workspace;
    rope_mode = 2;
  }
  // configurations 7 and 8: the software-pipelined kernel (4- and 8-wave
  // workgroups); RoPE on K per staged tile is not built into it and runs as
  // configuration 0
  if ((config == 7 || config == 8) && rope_mode != 1 && (in_dtype == ATTN_BF16 || in_dtype == ATTN_F16)) {
    launch_prefill_sp(p, in_dtype == ATTN_BF16, c, rope_mode == 2, config == 8 ? 2 : 1, stream);
    return attn_host::launch_status();
  }
  if ((config == 7 || config == 8) && in_dtype == ATTN_FP8_E5M2) {
    launch_prefill_sp8(p, c, stream);
    return attn_host::launch_status();
  }
  if (config == 7 || config == 8) config = 0;
  switch (in_dtype) {
    case ATTN_BF16:
      if (D == 64) launch_16bit<Bf16Tag, 64>(p, config, c, rope_mode, stream);
      else launch_16bit<Bf16Tag, 128>(p, config, c, rope_mode, stream);
      break;
    case ATTN_F16:
      if (D == 64) launch_16bit<F16Tag, 64>(p, config, c, rope_mode, stream);
      else launch_16bit<F16Tag, 128>(p, config, c, rope_mode, stream);
      break;
    default:  // fp8 e5m2 (RoPE rejected above): P in e4m3 on the fp8 MFMA; configuration 1: P in f16
      if (config == 1) {
        if (D == 64) launch_mfma<F16Tag, 64, true>(p, c, grid, stream);
        else launch_mfma<F16Tag, 128, true>(p, c, grid, stream);
      } else {
        if (D == 64) launch_mfma<F16Tag, 64, true, true>(p, c, grid, stream);
        else launch_mfma<F16Tag, 128, true, true>(p, c, grid, stream);
      }
      break;
  }
  return attn_host::launch_status();
}

// Tile configurations of the 16-bit MFMA prefill kernel (fp32 inputs have a
// single configuration; fp8 inputs use 1 for P in f16 and the default
// otherwise):
//   0: 4-wave workgroups (two per compute unit), 128 query rows, 64-key
//      tiles, one workgroup per work item (the fp8 default, and the kernel
//      for RoPE with K rotated per staged tile);
//   1: 8-wave workgroups whose two halves split the key tiles of 128 rows;
//   2: the tiling of 0, software-pipelined (S of the next tile overlaps the
//      softmax of this one);
//   3: the kernel of 0 with persistent scheduling once the work exceeds two
//      residency rounds: two resident workgroups per compute unit loop over
//      the items (snake order over the longest-first list); up to two rounds
//      it launches as 0.
//   4: the kernel of 0 with 32-key tiles: half the LDS and score registers,
//      three workgroups (three waves per SIMD) per compute unit, two
//      barriers per 64 keys (RoPE with K rotated per staged tile: as 0);
//   5: the workgroups of 1 with the two halves half a key tile apart, so
//      that one half's softmax overlaps the other's MFMAs (RoPE with K
//      rotated per staged tile: as 1);
//   6: the kernel of 0 with K and V tiles staged through registers instead
//      of LDS DMA (RoPE with K rotated per staged tile: as 0);
//   7 (global default for 16-bit inputs): the software-pipelined kernel
//      (prefill_sp.hip): 4-wave workgroups, the S MFMAs of the next key tile
//      interleaved with the softmax of this one and the PV MFMAs with the
//      rest of it, K/V tiles loaded an iteration ahead into per-stage LDS
//      arrays, causal items paired long with short in one workgroup (RoPE
//      with K rotated per staged tile: as 0);
//   8: the kernel of 7 with 8-wave workgroups whose halves take alternate key
//      tiles of the same rows (two waves per SIMD with half the items).
static const int kPrefillConfigs = 9;
static const int kPrefillGlobalConfig = 7;

extern "C" size_t attn_prefill_gqa_rope_workspace_bytes(int B, int Hkv, int S, int D, attn_dtype in_dtype,
                                                       float rope_theta) {
  if (B <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || !(rope_theta > 0.f)) return 0;
  if (in_dtype != ATTN_BF16 && in_dtype != ATTN_F16) return 0;  // fp32: own kernel; fp8: no RoPE
  return (size_t)B * Hkv * S * D * 2;  // rotated K, same layout as k
}

extern "C" attn_status attn_prefill_gqa_rope(const void* q, const void* k, const void* v, void* o,
                                             float* lse, int B, int Hq, int Hkv, int S, int D,
                                             attn_dtype in_dtype, attn_dtype out_dtype,
                                             float softmax_scale, int causal, float rope_theta,
                                             float q_descale, float k_descale, float v_descale,
                                             hipStream_t stream) {
  return prefill_impl(q, k, v, o, lse, B, Hq, Hkv, S, D, in_dtype, out_dtype, softmax_scale, causal,
                      rope_theta, q_descale, k_descale, v_descale, kPrefillGlobalConfig, nullptr, 0, false, stream);
}

extern "C" attn_status attn_prefill_gqa_rope_ws(const void* q, const void* k, const void* v, void* o,
                                                float* lse, int B, int Hq, int Hkv, int S, int D,
                                                attn_dtype in_dtype, attn_dtype out_dtype,
                                                float softmax_scale, int causal, float rope_theta,
                                                float q_descale, float k_descale, float v_descale,
                                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return prefill_impl(q, k, v, o, lse, B, Hq, Hkv, S, D, in_dtype, out_dtype, softmax_scale, causal,
                      rope_theta, q_descale, k_descale, v_descale, kPrefillGlobalConfig, workspace, workspace_bytes,
                      true, stream);
}

extern "C" attn_status attn_prefill_gqa_rope_with_config(
    const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int S,
    int D, attn_dtype in_dtype, attn_dtype out_dtype, float softmax_scale, int causal,
    float rope_theta, float q_descale, float k_descale, float v_descale, int config,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const bool k_rotated = (config & ATTN_CONFIG_K_ROTATED) != 0;
  config &= ~ATTN_CONFIG_K_ROTATED;
  if (config < 0 || config >= kPrefillConfigs) return ATTN_ERR_UNSUPPORTED;
  if (k_rotated && !workspace) return ATTN_ERR_WORKSPACE;
  return prefill_impl(q, k, v, o, lse, B, Hq, Hkv, S, D, in_dtype, out_dtype, softmax_scale, causal,
                      rope_theta, q_descale, k_descale, v_descale, config, workspace, workspace_bytes,
                      workspace != nullptr, stream, k_rotated);
}

extern "C" int attn_prefill_num_configs(void) { return kPrefillConfigs; }

// ---------------------------------------------------------------------------
// Chunked prefill against a cache prefix
// ---------------------------------------------------------------------------
// Keys per split: `split` if positive, else enough ranges that the launch has
// about 512 workgroups, with at least 256 keys per range (shorter ranges cost
// more in partial-result traffic than they gain in parallelism).
static int chunk_split_keys(int B, int Hq, int Hkv, int T, int cap, int split) {
  if (split > 0) return split;
  const int G = Hq / Hkv, GP = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const long long base = (long long)((T + 128 / GP - 1) / (128 / GP)) * B * Hkv * (G / GP);
  const long long want = (512 + base - 1) / base;
  long long keys = (cap + want - 1) / want;
  keys = (keys + 63) / 64 * 64;
  return (int)(keys < 256 ? 256 : keys);
}

extern "C" size_t attn_prefill_chunk_workspace_bytes(int B, int Hq, int Hkv, int T, int D, int cap, int split) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0 || D <= 0 || cap <= 0 || Hq % Hkv != 0) return 0;
  const int sk = chunk_split_keys(B, Hq, Hkv, T, cap, split);
  if (sk <= 0) return 0;
  const long long nsplit = (cap + sk - 1) / sk;
  if (nsplit <= 1) return 0;
  return split_workspace((long long)B * Hq * T, nsplit, D).total;
}

// chunk-mode launch: RoPE mode 2 (Q rotated in the kernel) or none
template <class Tag, int D>
static void launch_chunk_kernel(const PrefillParams& p, bool rope, dim3 grid, dim3 block, hipStream_t st) {
  if (rope) hipLaunchKernelGGL((prefill_fwd_kernel<Tag, D, true, 2, 1, true>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((prefill_fwd_kernel<Tag, D, true, 0, 1, true>), grid, block, 0, st, p);
}

// the chunk attention: kv_len[b] + kv_add keys per sequence; with k_new /
// v_new the kernel first writes the chunk's rows to the cache itself; `adv`,
// when given, advances kv_len once every reader is done (in the combine, or
// as a launch of its own when there is a single key range)
static attn_status chunk_attention(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_len,
                                   void* o, float* lse, void* workspace, size_t workspace_bytes, int B, int Hq,
                                   int Hkv, int T, int D, int cap, int split, attn_dtype dtype, attn_dtype out_dtype,
                                   float softmax_scale, float rope_theta, int kv_add, KvAdvance adv,
                                   hipStream_t stream, const void* k_new = nullptr, const void* v_new = nullptr) {
  if (!q || !k_cache || !v_cache || !kv_len || !o) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0 || D <= 0 || cap <= 0 || T > cap) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (split > 0 && (split % 64 != 0)) return ATTN_ERR_SHAPE;
  if (dtype < ATTN_F32 || dtype > ATTN_FP8_E5M2) return ATTN_ERR_DTYPE;
  if (out_dtype != ATTN_F32 && out_dtype != ATTN_F16 && out_dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (!(softmax_scale > 0.f) || !(softmax_scale < 3.0e38f)) return ATTN_ERR_SHAPE;
  if (rope_theta != rope_theta || !(rope_theta < 3.0e38f)) return ATTN_ERR_SHAPE;
  if (rope_theta > 0.f && cap > 65536) return ATTN_ERR_UNSUPPORTED;  // exact angle reduction needs pos < 2^16
  if (!attn_host::aligned(q, 16) || !attn_host::aligned(k_cache, 16) || !attn_host::aligned(v_cache, 16) ||
      !attn_host::aligned(o, 16) || !attn_host::aligned(kv_len, 4) || (lse && !attn_host::aligned(lse, 4)))
    return ATTN_ERR_ALIGN;
  if ((long long)B * Hkv * cap * D > (1LL << 40) || (long long)B * Hq * T * D > (1LL << 40)) return ATTN_ERR_SHAPE;

  const int sk = chunk_split_keys(B, Hq, Hkv, T, cap, split);
  const int nsplit = (cap + sk - 1) / sk;
  const long long R = (long long)B * Hq * T;
  SplitWorkspace w{};
  if (nsplit > 1) {
    w = split_workspace(R, nsplit, D);
    if (!workspace || workspace_bytes < w.total) return ATTN_ERR_WORKSPACE;
    if (!attn_host::aligned(workspace, 256)) return ATTN_ERR_ALIGN;
    if (R > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  }

  PrefillParams p{};
  p.q = q; p.k = k_cache; p.v = v_cache; p.o = o; p.lse = lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.S = T;
  p.G = Hq / Hkv;
  p.scale_log2 = softmax_scale * kLog2e;
  p.out_scale = 1.f;
  p.out_dtype = out_dtype;
  p.halves = 1;
  p.kv_len = kv_len;
  p.kv_add = kv_add;
  p.k_new = k_new;
  p.v_new = v_new;
  p.cap = cap;
  p.nsplit = nsplit;
  p.split_keys = sk;
  if (nsplit > 1) {
    p.ws_o = reinterpret_cast<float*>(workspace);
    p.ws_lse = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + w.lse_offset);
  }
  p.GP = (p.G % 4 == 0) ? 4 : (p.G % 2 == 0) ? 2 : 1;
  p.P = 128 / p.GP;
  p.n_ptiles = (T + p.P - 1) / p.P;
  p.n_hgroups = p.G / p.GP;
  const long long items = (long long)p.n_ptiles * B * Hkv * p.n_hgroups * nsplit;
  if (items > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  const dim3 grid((unsigned)items), block(256);
  const bool rope = rope_theta > 0.f;
  if (rope) {
    p.rope = 2;
    attn_host::rope_freq_split(rope_theta, D, p.inv_freq, p.rope_fhi, p.rope_flo);
    if (k_new) {  // the append kernel's three-part split for the keys (the same f_hi)
      float fhi3[64];
      attn_host::rope_freq_split(rope_theta, D, nullptr, fhi3, p.rope_flo3, p.rope_fmid);
    }
  }
  if (dtype == ATTN_BF16) {
    if (D == 64) launch_chunk_kernel<Bf16Tag, 64>(p, rope, grid, block, stream);
    else launch_chunk_kernel<Bf16Tag, 128>(p, rope, grid, block, stream);
  } else {
    if (D == 64) launch_chunk_kernel<F16Tag, 64>(p, rope, grid, block, stream);
    else launch_chunk_kernel<F16Tag, 128>(p, rope, grid, block, stream);
  }
  if (nsplit > 1 && ATTN_CHUNK_BF16_PARTS)
    launch_combine_bf16_parts(reinterpret_cast<const uint16_t*>(p.ws_o), p.ws_lse, o, (int)R, nsplit, D, out_dtype,
                              stream, lse, adv);
  else if (nsplit > 1) launch_combine(p.ws_o, p.ws_lse, o, (int)R, nsplit, D, out_dtype, stream, lse, adv);
  else if (adv.kv_len) launch_kv_advance(adv, stream);
  return attn_host::launch_status();
}

extern "C" attn_status attn_prefill_chunk(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* kv_len, void* o, float* lse, void* workspace,
                                          size_t workspace_bytes, int B, int Hq, int Hkv, int T, int D,
                                          int cap, int split, attn_dtype dtype, attn_dtype out_dtype,
                                          float softmax_scale, float rope_theta, hipStream_t stream) {
  return chunk_attention(q, k_cache, v_cache, kv_len, o, lse, workspace, workspace_bytes, B, Hq, Hkv, T, D, cap,
                         split, dtype, out_dtype, softmax_scale, rope_theta, 0, KvAdvance{}, stream);
}

extern "C" attn_status attn_prefill_chunk_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                               void* v_cache, int32_t* kv_len, void* o, float* lse,
                                               void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                                               int T, int D, int cap, int split, attn_dtype dtype,
                                               attn_dtype out_dtype, float softmax_scale, float rope_theta,
                                               hipStream_t stream) {
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !kv_len || !o) return ATTN_ERR_NULL;
  // the attention's checks first (they cover every shape the append takes),
  // so that a rejected call changes nothing
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0 || D <= 0 || cap <= 0 || T > cap || Hq % Hkv != 0)
    return ATTN_ERR_SHAPE;
  if (split > 0 && (split % 64 != 0)) return ATTN_ERR_SHAPE;
  if (dtype < ATTN_F32 || dtype > ATTN_FP8_E5M2) return ATTN_ERR_DTYPE;
  if (out_dtype != ATTN_F32 && out_dtype != ATTN_F16 && out_dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (!(softmax_scale > 0.f) || !(softmax_scale < 3.0e38f)) return ATTN_ERR_SHAPE;
  if (rope_theta != rope_theta || !(rope_theta < 3.0e38f)) return ATTN_ERR_SHAPE;
  if (rope_theta > 0.f && cap > 65536) return ATTN_ERR_UNSUPPORTED;
  if (!attn_host::aligned(q, 16) || !attn_host::aligned(k_new, 16) || !attn_host::aligned(v_new, 16) ||
      !attn_host::aligned(k_cache, 16) || !attn_host::aligned(v_cache, 16) || !attn_host::aligned(o, 16) ||
      !attn_host::aligned(kv_len, 4) || (lse && !attn_host::aligned(lse, 4)))
    return ATTN_ERR_ALIGN;
  if ((long long)B * Hkv * cap * D > (1LL << 40) || (long long)B * Hq * T * D > (1LL << 40) ||
      (long long)Hq * T * D > (1LL << 30))
    return ATTN_ERR_SHAPE;
  {
    const int sk = chunk_split_keys(B, Hq, Hkv, T, cap, split);
    const int nsplit = (cap + sk - 1) / sk;
    const long long R = (long long)B * Hq * T;
    if (nsplit > 1) {
      const SplitWorkspace w = split_workspace(R, nsplit, D);
      if (!workspace || workspace_bytes < w.total) return ATTN_ERR_WORKSPACE;
      if (!attn_host::aligned(workspace, 256)) return ATTN_ERR_ALIGN;
      if (R > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    }
    const int G = Hq / Hkv, GP = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1, P = 128 / GP;
    if ((long long)((T + P - 1) / P) * B * Hkv * (G / GP) * nsplit > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  }
  // chunks of up to 32 rows: the attention kernel writes the chunk's K
  // (rotated) and V to the cache itself; longer ones are appended first by
  // the append kernel (kv_len unchanged)
  const bool fused = T <= 32;
  if (!fused) {
    const attn_status st = attn_kv_append(k_new, v_new, nullptr, k_cache, v_cache, kv_len, B, Hkv, 0, T, D, cap,
                                          dtype, rope_theta, 0, stream);
    if (st != ATTN_OK) return st;
  }
  // the attention over kv_len + T keys, then the combine, which also
  // advances kv_len by T
  return chunk_attention(q, k_cache, v_cache, kv_len, o, lse, workspace, workspace_bytes, B, Hq, Hkv, T, D, cap,
                         split, dtype, out_dtype, softmax_scale, rope_theta, T, KvAdvance{kv_len, B, T, cap},
                         stream, fused ? k_new : nullptr, fused ? v_new : nullptr);
}
