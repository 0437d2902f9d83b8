// Software-pipelined prefill attention kernel for fp8 e5m2 inputs (D = 64 or
// 128) on gfx950: the fp8 counterpart of the 16-bit pipelined kernel, with
// both products on the 32x32x64 fp8 MFMA (twice the 16-bit rate).
//
// Operation: scaled-dot-product attention with online softmax on fp8 Q, K, V
// (persistent-attention digest, benchmark section: the forward pass in fp8
// e5m2); the probabilities go into the PV product rounded to fp8 e4m3, and
// the row sums are taken from the same rounded values, so the normalisation
// matches what was multiplied into V.
//
// Work split as in the 16-bit kernels: a workgroup of 4 waves (one per SIMD,
// one workgroup per compute unit) takes 128 query rows of one KV group, each
// wave 32 rows; scores are computed transposed (S^T = K Q^T), so a lane holds
// 32 keys of one query row and the pair of lanes l, l ^ 32 holds the row.
//
// What differs from the 16-bit kernel:
//   * K and V stay as their fp8 bytes in LDS (half the bytes per tile).  The
//     V^T operand comes from transposing 8-bit LDS reads (8 keys of one
//     column per lane), in the key order of the score accumulator, so the
//     probabilities need no shuffle between the two products.
//   * A PV MFMA spans all 64 keys of a tile, so it needs the whole tile's
//     probabilities: iteration i computes S(i+1), the exponentials of tile i
//     and PV(i-1).  A reference move decided after tile i+1's maximum is
//     applied to O after PV(i) has been added (the pending factor), since
//     P(i) was made with the old reference.
//   * The scale is not folded into Q (rounding a scaled Q to fp8 again would
//     add error; the MFMA's own scales are powers of two): each score takes
//     one multiply-add (s * scale - reference) before exp2.
//   * The row sums come from one more MFMA per tile (a block of ones times
//     P^T), not from vector adds.
// The running reference moves only when a row's tile maximum exceeds it by
// more than 2^8 (lazy rescaling, exact; probabilities stay below 256, inside
// the e4m3 range).

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "prefill_common.hpp"

namespace attn {

template <int N>
using ic8 = std::integral_constant<int, N>;
typedef __attribute__((ext_vector_type(2))) int i32x2;

// K and V^T fragments are read from LDS this many MFMAs ahead of their use
#ifndef ATTN_SP8_KPF
#define ATTN_SP8_KPF 1
#endif
#ifndef ATTN_SP8_VPF
#define ATTN_SP8_VPF 2
#endif

// max of three floats in one instruction.  (Through fmaxf the compiler
// first quiets possible signalling NaNs of every score that came through
// the mask's select, one extra instruction per score; scores here are never
// NaN: the MFMA of finite fp8 inputs is finite, masked ones are -inf.)
__device__ inline float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// 16-bit O through LDS, for whole-row stores (1: on), and the cache policy
// of those stores (16: sc1, device scope)
#ifndef ATTN_SP8_OLDS
#define ATTN_SP8_OLDS 1
#endif
#ifndef ATTN_SP8_OAUX
#define ATTN_SP8_OAUX 16
#endif

// NS: LDS stages per tensor; WPC: workgroups per compute unit the register
// allocation is made for (2: two waves per SIMD, at most 256 registers each)
template <int D, bool CAUSAL, int NS, int WPC>
__global__ __launch_bounds__(256, WPC) void prefill_sp8_kernel(const PrefillParams p) {
  static_assert(NS == 2 || NS == 4, "2 or 4 LDS stages per tensor (score tiles alternate by parity)");
  constexpr int BN = 64;              // keys per tile
  constexpr int NB = BN / 32;         // 32-key blocks of a score tile
  constexpr int ROWB = D;             // bytes per K/V row
  constexpr int CH = D / 16;          // 16-byte chunks per row
  constexpr int TILEB = BN * ROWB;    // bytes of one K or V tile
  constexpr int RPI = 64 / CH;        // rows per wave-wide DMA instruction
  constexpr int IPW = BN / RPI / 4;   // DMA instructions per wave per tile and tensor
  constexpr int NU = D / 64;          // 64-deep k-steps of a score block
  constexpr int NDB = D / 32;         // 32-wide d blocks of O
  constexpr int NJS = NB * NU;        // S MFMAs per tile
  constexpr int NJV = NDB + 1;        // PV MFMAs per tile, plus the row-sum MFMA
  constexpr int NC = NJS + NJV;       // MFMA chunks per iteration
  constexpr int NE = 8;               // probability dwords per lane (4 scores each)
  constexpr float kLazy = 8.f;

  __shared__ __attribute__((aligned(1024))) uint8_t k0[TILEB], k1[TILEB], k2[NS > 2 ? TILEB : 16],
      k3[NS > 3 ? TILEB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t v0[TILEB], v1[TILEB], v2[NS > 2 ? TILEB : 16],
      v3[NS > 3 ? TILEB : 16];
  // stage of tile t: t mod NS (for K and V alike)
  auto kst = [&](auto s) -> uint8_t* {
    constexpr int t = ((decltype(s)::value % NS) + NS) % NS;
    if constexpr (t == 0) return k0;
    else if constexpr (t == 1) return k1;
    else if constexpr (t == 2) return k2;
    else return k3;
  };
  auto vst = [&](auto s) -> uint8_t* {
    constexpr int t = ((decltype(s)::value % NS) + NS) % NS;
    if constexpr (t == 0) return v0;
    else if constexpr (t == 1) return v1;
    else if constexpr (t == 2) return v2;
    else return v3;
  };

  // XOR swizzles of the 16-byte chunks of a row for the 64-bank LDS.  K is
  // read 16 rows at one chunk per 16 lanes; V is read transposed, 8 rows of
  // 16 bytes per 16 lanes, keys {0-3, 8-11} (+4 in the upper half-wave).
  auto kswz = [](int row) { return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3); };
  auto vswz = [](int row) { return D == 128 ? 2 * ((row >> 1) & 1) + 4 * ((row >> 3) & 1) : 2 * ((row >> 3) & 1); };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, hh = lane >> 5;
  const int g = lane >> 4, li = lane & 15;

  // K A operand of block nb, k-step u: row 32 nb + m, bytes 64 u + 32 hh .. +31
  // (logical chunks 4 u + 2 hh and 4 u + 2 hh + 1)
  int koff[NU][2];
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h) koff[u][h] = m * ROWB + 16 * ((4 * u + 2 * hh + h) ^ kswz(m));
  // V^T A operand of d block db: 4 transposing reads q = 0..3, each giving 8
  // keys of column d = 32 db + m.  In a 16-lane group, lane 2r + b names row
  // r (byte r of every lane's result) at columns 8b .. 8b+7 of the group's 16
  // columns.  Byte r of read q must be the key whose probability sits in the
  // same byte of the P^T operand: key 16 q + 8 (r / 4) + 4 hh + r % 4.
  int voff[NDB];
  {
    const int r = li >> 1, b8 = li & 1;
    const int key = 8 * (r >> 2) + 4 * hh + (r & 3);  // + 16 q per read
#pragma unroll
    for (int db = 0; db < NDB; ++db) voff[db] = key * ROWB + 16 * ((2 * db + (g & 1)) ^ vswz(key)) + 8 * b8;
  }
  int dk[IPW], dv[IPW];  // DMA source offsets (row inside the tile, swizzled chunk)
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int row = RPI * (wave * IPW + u) + lane / CH, phys = lane % CH;
    dk[u] = row * ROWB + 16 * (phys ^ kswz(row));
    dv[u] = row * ROWB + 16 * (phys ^ vswz(row));
  }

  const int wg = blockIdx.x;
  // causal pairs, grouped by head: workgroup w = r hp + j takes query tiles
  // n_ptiles - 1 - j and j of head group r (a long and a short item, the
  // same amount of work in every workgroup; the pairs in flight share the
  // K/V of a few heads)
  // With a head count that is a multiple of 8 the order is also XCD-aware:
  // workgroups are dealt to the 8 XCDs in turn (w mod 8), so head r goes to
  // XCD r mod 8 and each XCD takes its heads one after another, keeping a
  // head's K/V in one L2.  Non-causal items are all equally long and go
  // head-major the same way.
  const int heads = p.B * p.Hkv * p.n_hgroups;
  const int hp = (p.n_ptiles + 1) / 2;
  const bool xcd = heads % 8 == 0;
  const int wx = xcd ? (wg & 7) : 0, wi = xcd ? wg >> 3 : wg;  // XCD, index on it
  const int per_head = CAUSAL ? hp : p.n_ptiles;
  const int pr = xcd ? (wi / per_head) * 8 + wx : wi / per_head;  // head group
  const int pj = wi % per_head;                                    // pair / query tile of it
  const int n_my = CAUSAL ? (p.n_ptiles - 1 - pj > pj ? 2 : 1) : 1;
  const float c = p.scale_log2;
  i32x8 ones = {0x3c3c3c3c, 0x3c3c3c3c, 0x3c3c3c3c, 0x3c3c3c3c,
                0x3c3c3c3c, 0x3c3c3c3c, 0x3c3c3c3c, 0x3c3c3c3c};  // e5m2 1.0
  asm volatile("" : "+v"(ones));  // kept in registers, not rebuilt before every use

#pragma unroll 1
  for (int itn = 0; itn < n_my; ++itn) {
    if (itn > 0) asm volatile("s_barrier" ::: "memory");
    const int ptile = CAUSAL ? (itn == 0 ? p.n_ptiles - 1 - pj : pj) : pj;
    int rest = pr;
    const int hg = rest % p.n_hgroups;
    rest /= p.n_hgroups;
    const int kvh = rest % p.Hkv;
    const int b = rest / p.Hkv;
    const int head = kvh * p.G + hg * p.GP + (wave % p.GP);
    const int p0 = ptile * p.P;
    const int pw0 = p0 + (wave / p.GP) * 32;
    const int qpos = pw0 + m;
    const int kend = CAUSAL ? min(p.S, p0 + p.P) : p.S;
    const int n_kt = (kend + BN - 1) / BN;
    const int n_w = pw0 >= p.S ? 0 : CAUSAL ? min(n_kt, min(pw0 + 31, p.S - 1) / BN + 1) : n_kt;

    const size_t kv_row0 = ((size_t)b * p.Hkv + kvh) * p.S;
    const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.k) + kv_row0 * ROWB;
    const uint8_t* vg = reinterpret_cast<const uint8_t*>(p.v) + kv_row0 * ROWB;
    // buffer range of key tile t: ends at the sequence end; tiles before the
    // first (t < 0) and past the end have an empty range, so their loads
    // write zeros without touching memory.  Every tile issues the same number
    // of loads (exact vmcnt arithmetic).
    auto tile_rsrc = [&](const uint8_t* src, int t) {
      const int key0 = t * BN;
      const int range = t < 0 ? 0 : max(0, p.S - key0) * ROWB;
      const int kb = t < 0 ? 0 : min(key0, p.S);
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src + (size_t)kb * ROWB), (short)0, range,
                                               kBufferRsrcWord3);
    };
    auto dma1 = [&](__amdgpu_buffer_rsrc_t rs, uint8_t* dst, const int* loff, int u) {
      int wrow = wave * (RPI * IPW * ROWB);
      asm volatile("" : "+s"(wrow));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_AS(void, dst + wrow + RPI * u * ROWB), 16, loff[u], 0, 0, 0);
    };
    auto dma = [&](const uint8_t* src, uint8_t* dst, const int* loff, int t) {
      const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src, t);
#pragma unroll
      for (int u = 0; u < IPW; ++u) dma1(rs, dst, loff, u);
    };

    // ---- Q fragments (B operand of S^T = K Q^T): bytes 64 u + 32 hh .. +31 ----
    uint32_t qf[NU * 8];
    {
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(p.q) + (((size_t)b * p.Hq + head) * p.S + qpos) * D;
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 w = qpos < p.S ? ldg16(qrow + 64 * u + 32 * hh + 16 * h) : u32x4{0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 4; ++e) qf[8 * u + 4 * h + e] = w[e];
        }
    }
    // loads: K(0), then one batch per pipeline slot bi = 0 .. NS-2:
    // {K(bi + 1), V(bi - 1)} (V(-1) is an empty range: zeros)
    dma(kg, kst(ic8<0>{}), dk, 0);
    auto prologue_batch = [&](auto bb) {
      constexpr int bi = decltype(bb)::value;
      dma(kg, kst(ic8<bi + 1>{}), dk, bi + 1);
      dma(vg, vst(ic8<bi - 1>{}), dv, bi - 1);
    };
    prologue_batch(ic8<0>{});
    if constexpr (NS > 2) prologue_batch(ic8<1>{});
    if constexpr (NS > 3) prologue_batch(ic8<2>{});
    auto qfrag = [&](int u) {
      return i32x8{(int)qf[8 * u], (int)qf[8 * u + 1], (int)qf[8 * u + 2], (int)qf[8 * u + 3],
                   (int)qf[8 * u + 4], (int)qf[8 * u + 5], (int)qf[8 * u + 6], (int)qf[8 * u + 7]};
    };

    // ---- running state ----
    f32x16 acc_o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
    f32x16 acc_l = {};        // row sums (every entry of a lane: its row's sum)
    f32x16 sA[NB], sB[NB];    // raw score tiles of even / odd key tiles
    uint32_t pA[NE], pB[NE];  // e4m3 probabilities of even / odd key tiles (P^T B operand)
#pragma unroll
    for (int w = 0; w < NE; ++w) pA[w] = pB[w] = 0u;
    float m_ref = 0.f;        // reference (exponent domain), equal in both lanes of a row
    float alpha = 1.f;        // pending factor for O and the row sums (see above)
    bool pend = false;        // wave-uniform: a factor is pending

    auto krd = [&](const uint8_t* kb, int j) {
      const int nb = j / NU, u = j % NU;
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(kb + koff[u][0] + 32 * nb * ROWB);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(kb + koff[u][1] + 32 * nb * ROWB);
      return i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    };
    auto vrd = [&](const uint8_t* vb, int db) {
      i32x8 r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_AS(i32x2, vb + voff[db] + 16 * q * ROWB));
        r[2 * q] = x[0];
        r[2 * q + 1] = x[1];
      }
      return r;
    };
    auto needs_mask = [&](int t) {
      const int key0 = t * BN;
      return (key0 + BN > p.S) || (CAUSAL && key0 + BN - 1 > pw0);
    };
    auto mask = [&](f32x16* s, int t) {
      const int lim = (CAUSAL ? min(qpos, p.S - 1) : p.S - 1) - t * BN - 4 * hh;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * nb + 8 * (r >> 2) + (r & 3) > lim) s[nb][r] = kNegInf;
    };
    // Probability dword w of a tile holds k-slots 4w .. 4w+3 of the lane
    // (score block w / 4, values 4 (w % 4) .. +3).  Its four exponentials
    // are taken in the chunk ce(w) and rounded / packed one chunk later (no
    // in-order issue stall on the exp results).  Chunks 0 .. NJS-1 are the S
    // MFMAs, NJS .. NC-1 the PV MFMAs and the row-sum MFMA.
    auto ce = [](int w) { return w * NC / NE; };
    float ex[NE][4];
    auto expw = [&](const f32x16* s, int w) {
      const float nm = -m_ref;
#pragma unroll
      for (int t = 0; t < 4; ++t) ex[w][t] = fast_exp2(fmaf(s[w / 4][4 * (w % 4) + t], c, nm));
    };
    auto packw = [&](uint32_t* pd, int w) {
      // (the low half is written first; the register's old contents, the
      // dword of two tiles back, are all replaced)
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(ex[w][0], ex[w][1], (int)pd[w], false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(ex[w][2], ex[w][3], v, true);
      pd[w] = (uint32_t)v;
    };
    // VALU share of chunk j: exponentials and packing of tile `sp` into pd
    auto softmax_share = [&](int j, const f32x16* sp, uint32_t* pd) {
#pragma unroll
      for (int w = 0; w < NE; ++w) {
        if (ce(w) == j) expw(sp, w);
        if (ce(w) + 1 == j) packw(pd, w);
      }
    };

    // S of the tile in stage stc into s (raw scores), with the softmax share
    // of tile sp and (if `loads`) the K loads of this iteration
    auto s_phase = [&](auto stc, f32x16* s, const f32x16* sp, uint32_t* pd, bool loads, __amdgpu_buffer_rsrc_t krs,
                       uint8_t* kdst) {
      const uint8_t* kb = kst(stc);
      constexpr int KPF = ATTN_SP8_KPF < NJS ? ATTN_SP8_KPF : NJS;
      i32x8 fa[KPF + 1];
#pragma unroll
      for (int x = 0; x < KPF; ++x) fa[x] = krd(kb, x);
#pragma unroll
      for (int j = 0; j < NJS; ++j) {
        if (j + KPF < NJS) fa[(j + KPF) % (KPF + 1)] = krd(kb, j + KPF);
        const int nb = j / NU, u = j % NU;
        s[nb] = mfma32_bf8(fa[j % (KPF + 1)], qfrag(u), u == 0 ? f32x16{} : s[nb]);
        if (sp) softmax_share(j, sp, pd);
        if (loads) {
#pragma unroll
          for (int uu = 0; uu < IPW; ++uu)
            if (j == (NJS > IPW ? 1 : 0) + uu) dma1(krs, kdst, dk, uu);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // PV of the tile in stage stc with probabilities pp (and its row sums),
    // with the rest of the softmax share of tile sp, the row maximum of the
    // next score tile sn and (if `loads`) the V loads of this iteration.
    // Returns the raw row maximum of sn (both lanes of the pair).
    auto pv_phase = [&](auto stc, const uint32_t* pp, const f32x16* sp, uint32_t* pd, const f32x16* sn, bool loads,
                        __amdgpu_buffer_rsrc_t vrs, uint8_t* vdst) {
      const uint8_t* vb = vst(stc);
      constexpr int VPF = ATTN_SP8_VPF < NDB ? ATTN_SP8_VPF : NDB;
      i32x8 fv[VPF + 1];
#pragma unroll
      for (int x = 0; x < VPF; ++x) fv[x] = vrd(vb, x);
      const i32x8 pb = {(int)pp[0], (int)pp[1], (int)pp[2], (int)pp[3], (int)pp[4], (int)pp[5], (int)pp[6], (int)pp[7]};
      float mx = kNegInf, mx2 = kNegInf;
#pragma unroll
      for (int j = 0; j < NJV; ++j) {
        if (j + VPF < NDB) fv[(j + VPF) % (VPF + 1)] = vrd(vb, j + VPF);
        if (j < NDB) acc_o[j] = mfma32_bf8_fp8(fv[j % (VPF + 1)], pb, acc_o[j]);
        else acc_l = mfma32_bf8_fp8(ones, pb, acc_l);
        if (sp) softmax_share(NJS + j, sp, pd);
        if (sn) {
#pragma unroll
          for (int k2 = 0; k2 < 16; ++k2) {  // max3 over value pair k2 of the next tile
            if (k2 * NJV / 16 == j) {
              const float a = sn[k2 / 8][(2 * k2) % 16], a2 = sn[k2 / 8][(2 * k2) % 16 + 1];
              if (k2 & 1) mx2 = max3(mx2, a, a2);
              else mx = max3(mx, a, a2);
            }
          }
          asm volatile("" : "+v"(mx), "+v"(mx2));
        }
        if (loads) {
#pragma unroll
          for (int uu = 0; uu < IPW; ++uu)
            if (j == 1 + uu) dma1(vrs, vdst, dv, uu);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (sp) softmax_share(NC, sp, pd);  // packing of the last chunk's exponentials
      return pair_max32(fmaxf(mx, mx2));
    };

    // ---- prologue: S of tile 0 and the initial reference ----
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * IPW * (NS - 1)));  // K(0) of this wave landed
    asm volatile("s_barrier" ::: "memory");                      // ... and of every wave
    {
      s_phase(ic8<0>{}, sA, nullptr, nullptr, false, tile_rsrc(kg, 0), nullptr);
      if (needs_mask(0)) mask(sA, 0);
      float mx = kNegInf;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sA[nb][r]);
      mx = pair_max32(mx);
      m_ref = mx == kNegInf ? 0.f : mx * c;
    }

    // ---- key loop: iterations i = 0 .. n_kt (the last one only finishes
    // PV(n_kt - 1); the tiles it scores lie past the end, fully masked).
    // Iteration i: wait for K(i+1) and V(i-1) (the batch issued NS - 1
    // iterations earlier) and the barrier; issue K(i + NS) into the stage of
    // K(i) and V(i + NS - 2) into the stage of V(i - 2), both read by every
    // wave before this barrier; then
    //   S(i+1) MFMAs          || exponentials of tile i (first part)
    //   mask S(i+1)
    //   PV(i-1), row sums     || exponentials of tile i (rest), max of S(i+1)
    //   apply the pending factor (O now holds tiles up to i-1, in the units
    //   of the reference P(i-1) was made with)
    //   move the reference if a row's maximum grew by more than 2^8; the
    //   factor waits until PV(i) is in. ----
    auto iter = [&](auto phc, int i) {
      constexpr int PH = decltype(phc)::value;  // i % NS
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * IPW * (NS - 2)));
      asm volatile("s_barrier" ::: "memory");
      f32x16* sc = (PH & 1) ? sB : sA;  // S(i)
      f32x16* sn = (PH & 1) ? sA : sB;  // S(i+1)
      uint32_t* pc = (PH & 1) ? pB : pA;  // P(i)
      uint32_t* pp = (PH & 1) ? pA : pB;  // P(i-1)
      s_phase(ic8<PH + 1>{}, sn, sc, pc, true, tile_rsrc(kg, i + NS), kst(ic8<PH>{}));
      // the exponentials made so far stay ahead of the mask branch
#pragma unroll
      for (int w = 0; w < NE; ++w)
        if (ce(w) < NJS) asm volatile("" ::"v"(ex[w][0]), "v"(ex[w][1]), "v"(ex[w][2]), "v"(ex[w][3]));
      if (needs_mask(i + 1)) mask(sn, i + 1);
      const float mx = pv_phase(ic8<PH + NS - 1>{}, pp, sc, pc, sn, true, tile_rsrc(vg, i + NS - 2),
                                vst(ic8<PH + NS - 2>{}));
      if (pend) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
        acc_l *= alpha;
        pend = false;
      }
      const float d = mx * c - m_ref;
      if (__ballot(d > kLazy)) {
        const float dd = fmaxf(d, 0.f);
        alpha = fast_exp2(-dd);
        m_ref += dd;
        pend = true;
      }
    };
    const int n_it = n_kt + 1;
#pragma unroll 1
    for (int i0 = 0; i0 < n_it; i0 += NS) {
      iter(ic8<0>{}, i0);
      if (i0 + 1 >= n_it) break;
      iter(ic8<1>{}, i0 + 1);
      if constexpr (NS > 2) {
        if (i0 + 2 >= n_it) break;
        iter(ic8<2>{}, i0 + 2);
      }
      if constexpr (NS > 3) {
        if (i0 + 3 >= n_it) break;
        iter(ic8<3>{}, i0 + 3);
      }
    }

    // ---- epilogue: O / l (the last iteration's reference move, decided on
    // masked tiles, never happens: its maximum is -inf) ----
    const float l = acc_l[0];
    const float inv = l > 0.f ? p.out_scale / l : 0.f;
#if ATTN_SP8_OLDS
    if (p.out_dtype != ATTN_F32) {
      // 16-bit O leaves through LDS, so that every store instruction writes
      // 16-byte pieces of whole rows (a lane's accumulator holds 4-element
      // pieces of one row: stored directly, each instruction touches 32
      // rows).  Wave w transposes through stage array w (a 64-key fp8 tile
      // holds exactly 32 rows of 16-bit output) once every wave is past its
      // key loop and the loads into the stages have landed; the barrier at
      // the start of the next item keeps that item's loads out until all
      // waves have read their rows back.
      uint8_t* area = wave == 0 ? k0 : wave == 1 ? k1 : wave == 2 ? v0 : v1;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      asm volatile("s_barrier" ::: "memory");
      if (n_w > 0) {
        int lm = m, ln = lane;
        asm volatile("" : "+v"(lm), "+v"(ln));  // keep the addresses below out of the item loop
        auto stage_out = [&](auto odt) {
          constexpr int OD = decltype(odt)::value;
          constexpr int RB = D * 2;        // bytes per output row
          constexpr int CPR = RB / 16;     // 16-byte pieces per row (XOR-swizzled by row)
          constexpr int RPR = 64 / CPR;    // rows per read instruction
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int byte = (32 * db + 8 * g4 + 4 * hh) * 2;
              uint8_t* dst = area + lm * RB + 16 * ((byte / 16) ^ (lm % CPR)) + byte % 16;
              const float o0 = acc_o[db][4 * g4] * inv, o1 = acc_o[db][4 * g4 + 1] * inv;
              const float o2 = acc_o[db][4 * g4 + 2] * inv, o3 = acc_o[db][4 * g4 + 3] * inv;
              if constexpr (OD == ATTN_BF16) *reinterpret_cast<u32x2*>(dst) = u32x2{Bf16Tag::pack2(o0, o1), Bf16Tag::pack2(o2, o3)};
              else *reinterpret_cast<u32x2*>(dst) = u32x2{F16Tag::pack2(o0, o1), F16Tag::pack2(o2, o3)};
            }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's LDS writes are done before its reads
          // all reads first, then all stores; the buffer range ends at the
          // sequence end, so rows past it are dropped without a branch
          // (the base is moved to scalar registers explicitly: built from
          // values the compiler had placed in vector registers, the buffer
          // descriptor would be wrapped in a loop over its distinct values)
          const uint64_t oa = reinterpret_cast<uint64_t>(reinterpret_cast<uint8_t*>(p.o) +
                                                         (((size_t)b * p.Hq + head) * p.S + pw0) * RB);
          uint8_t* obase = reinterpret_cast<uint8_t*>(
              ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(oa >> 32)) << 32) |
              (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)oa));
          const int orange = __builtin_amdgcn_readfirstlane(max(0, min(p.S - pw0, 32)) * RB);
          const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(obase, (short)0, orange, kBufferRsrcWord3);
          u32x4 ov[32 / RPR];
#pragma unroll
          for (int i = 0; i < 32 / RPR; ++i) {
            const int r = RPR * i + ln / CPR, c = ln % CPR;
            ov[i] = *reinterpret_cast<const u32x4*>(area + r * RB + 16 * (c ^ (r % CPR)));
          }
#pragma unroll
          for (int i = 0; i < 32 / RPR; ++i)
            __builtin_amdgcn_raw_buffer_store_b128(ov[i], ors, (RPR * i + ln / CPR) * RB + 16 * (ln % CPR), 0,
                                                   ATTN_SP8_OAUX);
        };
        if (p.out_dtype == ATTN_BF16) stage_out(ic8<ATTN_BF16>{});
        else stage_out(ic8<ATTN_F16>{});
        if (p.lse && hh == 0 && qpos < p.S)
          p.lse[((size_t)b * p.Hq + head) * p.S + qpos] = l > 0.f ? (m_ref + __log2f(l)) * kLn2 : kNegInf;
      }
    } else
#endif
    if (qpos < p.S && n_w > 0) {
      const size_t row = ((size_t)b * p.Hq + head) * p.S + qpos;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int r = 4 * g4;
          store4(p.o, row * D + 32 * db + 8 * g4 + 4 * hh, p.out_dtype, acc_o[db][r] * inv, acc_o[db][r + 1] * inv,
                 acc_o[db][r + 2] * inv, acc_o[db][r + 3] * inv);
        }
      if (p.lse && hh == 0) p.lse[row] = l > 0.f ? (m_ref + __log2f(l)) * kLn2 : kNegInf;
    }
  }
}

// D = 128: two stages and two workgroups per compute unit (two waves per
// SIMD; 32 KB of LDS each); D = 64: four stages, one workgroup per compute
// unit (measured: a second wave per SIMD gains nothing there)
#ifndef ATTN_SP8_NS128
#define ATTN_SP8_NS128 2
#endif
#ifndef ATTN_SP8_WPC128
#define ATTN_SP8_WPC128 2
#endif
#ifndef ATTN_SP8_NS64
#define ATTN_SP8_NS64 4
#endif
#ifndef ATTN_SP8_WPC64
#define ATTN_SP8_WPC64 1
#endif
template <int D, bool CAUSAL>
static void launch_sp8_t(const PrefillParams& p, hipStream_t st) {
  const long long heads = (long long)p.B * p.Hkv * p.n_hgroups;
  const unsigned grid = (unsigned)(CAUSAL ? (p.n_ptiles + 1) / 2 * heads : p.n_ptiles * heads);
  constexpr int NS = D == 128 ? ATTN_SP8_NS128 : ATTN_SP8_NS64;
  constexpr int WPC = D == 128 ? ATTN_SP8_WPC128 : ATTN_SP8_WPC64;
  hipLaunchKernelGGL((prefill_sp8_kernel<D, CAUSAL, NS, WPC>), dim3(grid), dim3(256), 0, st, p);
}

void launch_prefill_sp8(const PrefillParams& p, bool causal, hipStream_t st) {
  if (p.D == 64) {
    if (causal) launch_sp8_t<64, true>(p, st);
    else launch_sp8_t<64, false>(p, st);
  } else {
    if (causal) launch_sp8_t<128, true>(p, st);
    else launch_sp8_t<128, false>(p, st);
  }
}

}  // namespace attn
