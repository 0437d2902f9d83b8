// Software-pipelined prefill attention kernel (16-bit inputs, D = 64 or 128)
// for gfx950: one wave per SIMD, the matrix work of one key tile overlapped
// with the softmax work of its neighbour inside each wave.
//
// Operation: the textbook scaled-dot-product attention with online softmax
// (shape-adaptive attention lesson page, rows "What was tried" and
// "Conditions": causal GQA prefill with RoPE fused into attention), with the
// same work split, LDS layouts and MFMA operand layouts as the 4-wave
// prefill kernel: a workgroup of 4 waves takes 128 query rows of one KV
// group (GQA heads side by side at the same positions), each wave 32 rows,
// scores computed transposed (S^T = K Q^T, one query row per lane pair).
//
// What is different:
//   * One workgroup per compute unit, one wave per SIMD, so a wave may hold
//     up to 512 registers and nothing else shares its SIMD.  The overlap of
//     matrix and vector work comes from the order of the wave's own
//     instruction stream: the S MFMAs of key tile i+1 are issued between the
//     exponentials of tile i, and the PV MFMAs of tile i between the row
//     maxima of tile i+1 (a wave issues VALU work while its MFMAs run).
//   * Scores arrive in the exponent domain already: Q is multiplied by
//     softmax_scale * log2(e) when its fragments are built (inside the RoPE
//     rotation, before the one rounding to the input type), and the first
//     MFMA of every score block accumulates onto -m (the row's running
//     reference, held in a register block), so exp2 takes the MFMA result
//     directly, with no per-score multiply-add.
//   * K and V stream HBM -> LDS by DMA (buffer loads with the LDS bit) NS
//     tiles ahead, into stages that are separate LDS arrays: reads of one
//     stage then only wait for the loads into that stage, not for every load
//     in flight.
//   * Causal launches pair work items k and n-1-k of the longest-first order
//     in one workgroup, so every workgroup does the same number of key tiles.
// The running reference moves only when a row's tile maximum exceeds it by
// more than 2^8 (lazy rescaling; exact, probabilities stay below 256).

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "prefill_common.hpp"

namespace attn {

template <int N>
using ic = std::integral_constant<int, N>;

// cache policy of the O stores: device scope (sc1).  Stores that leave no
// dirty lines in the XCD's L2 shorten its write-back at the end of the
// kernel (measured on the causal GQA RoPE prefill, S=2048: 0.7 us less per
// step; non-temporal sc1 measured the same)
#ifndef ATTN_SP_OAUX
#define ATTN_SP_OAUX 16
#endif
// LDS stages per tensor (K runs NS tiles ahead of its use, V NS - 1) and
// workgroups per compute unit the register allocation aims for
#ifndef ATTN_SP_STAGES
#define ATTN_SP_STAGES 2
#endif
#ifndef ATTN_SP_WG_PER_CU
#define ATTN_SP_WG_PER_CU 1
#endif
// 8-wave kernel: the halves run half an iteration apart (a second barrier
// per iteration between the S and the PV phase, the second half one barrier
// behind), so one half's S phase meets the other half's PV phase
#ifndef ATTN_SP_PINGPONG
#define ATTN_SP_PINGPONG 0
#endif
// causal launches: 1 = a workgroup takes items k and n-1-k in turn; 0 = one
// item per workgroup, workgroup n/2 + k taking the short item n-1-k (two
// workgroups share a compute unit, and k and n/2 + k tend to meet there)
#ifndef ATTN_SP_PAIR
#define ATTN_SP_PAIR 1
#endif
// MFMA operands are read from LDS this many MFMAs ahead of their use
#ifndef ATTN_SP_KPF
#define ATTN_SP_KPF 3
#endif
#ifndef ATTN_SP_VPF
#define ATTN_SP_VPF 2
#endif
// row sum of a packed pair of probabilities: 2 = the two fp32 values added
// before rounding (two adds that issue beside the MFMAs); 0 = one dot product
// of the rounded pair against ones (a dot product next to an MFMA stalls the
// wave for about half an MFMA); 1 = the two rounded halves widened and added
#ifndef ATTN_SP_LSUM
#define ATTN_SP_LSUM 2
#endif

// HALVES = 2: 8-wave workgroups whose two halves (4 waves each, one wave of
// each on every SIMD) take alternate key tiles of the same query rows, each
// half with its own LDS stages, and merge their results through LDS at the
// end of an item: two waves per SIMD where the work has too few items for
// two 4-wave workgroups per compute unit.
template <class Tag, int D, bool CAUSAL, bool RQ, int NS, int HALVES>
__global__ __launch_bounds__(256 * HALVES, ATTN_SP_WG_PER_CU) void prefill_sp_kernel(const PrefillParams p) {
  static_assert(NS == 2 || NS == 4, "2 or 4 LDS stages per tensor");
  static_assert(HALVES == 1 || HALVES == 2, "4 or 8 waves");
  constexpr int BN = 64;             // keys per tile
  constexpr int NB = BN / 32;        // 32-key blocks of a score tile
  constexpr int CPB = BN / 16;       // 16-key k-steps of the PV MFMAs
  constexpr int ROWB = D * 2;        // bytes per K/V row
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int TILEB = BN * ROWB;   // bytes of one K or V tile
  constexpr int RPI = 64 / CH;       // rows per wave-wide DMA instruction
  constexpr int IPW = BN / RPI / 4;  // DMA instructions per wave per tile and tensor
  constexpr int NKK = D / 16, NDB = D / 32;
  constexpr int NJS = NB * NKK;      // S MFMAs per tile
  constexpr int NJV = NDB * CPB;     // PV MFMAs per tile
  constexpr float kLazy = 8.f;

  // one array per stage (a read of one stage then waits only for the loads
  // into it), HALVES tiles each
  __shared__ __attribute__((aligned(1024))) uint8_t k0[HALVES * TILEB], k1[HALVES * TILEB],
      k2[NS > 2 ? HALVES * TILEB : 16], k3[NS > 2 ? HALVES * TILEB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t v0[HALVES * TILEB], v1[HALVES * TILEB],
      v2[NS > 2 ? HALVES * TILEB : 16], v3[NS > 2 ? HALVES * TILEB : 16];
  __shared__ __attribute__((aligned(16))) float rtab[RQ && HALVES == 1 ? D : 4];  // (after the stages)
  auto kst = [&](auto s) -> uint8_t* {
    constexpr int t = decltype(s)::value % NS;
    if constexpr (t == 0) return k0;
    else if constexpr (t == 1) return k1;
    else if constexpr (t == 2) return k2;
    else return k3;
  };
  auto vst = [&](auto s) -> uint8_t* {
    constexpr int t = decltype(s)::value % NS;
    if constexpr (t == 0) return v0;
    else if constexpr (t == 1) return v1;
    else if constexpr (t == 2) return v2;
    else return v3;
  };

  // XOR swizzles of the 16-byte chunks of a row for the 64-bank LDS (as in
  // the 4-wave kernel): K read by 16 consecutive rows at one chunk, V read
  // transposed as 4 rows x 4 chunks per 32 lanes
  auto kswz = [](int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); };
  auto vswz = [](int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: DMA addressing stays scalar
  const int wq = wave & 3;                                     // wave inside its half
  const int half = HALVES == 2 ? wave >> 2 : 0;
  const int hoff = half * TILEB;                               // this half's tile inside a stage
  const int m = lane & 31, hh = lane >> 5;
  const int g = lane >> 4, rr = lane & 15;

  int koff[NKK];  // K A operand: row 32 nb + m, logical chunk 2 kk + hh
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) koff[kk] = m * ROWB + 16 * ((2 * kk + hh) ^ kswz(m));
  int voff[NDB];  // V^T A operand by transposing reads (key order inside 16-key blocks matches the accumulator)
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d = 32 * db + 16 * (g & 1) + 4 * (rr & 3);
    const int key = 4 * (g >> 1) + (rr >> 2);
    voff[db] = key * ROWB + 16 * ((d >> 3) ^ vswz(key)) + 2 * (d & 7);
  }
  int dk[IPW], dv[IPW];  // DMA source offsets (row inside the tile, swizzled chunk)
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int row = RPI * (wq * IPW + u) + lane / CH, phys = lane % CH;
    dk[u] = row * ROWB + 16 * (phys ^ kswz(row));
    dv[u] = row * ROWB + 16 * (phys ^ vswz(row));
  }

  const int per_ptile = p.B * p.Hkv * p.n_hgroups;
  const int n_items = p.n_ptiles * per_ptile;
  const int wg = blockIdx.x;
  constexpr bool PAIR = CAUSAL && ATTN_SP_PAIR;
  // causal pairs, grouped by head: workgroup w = r hp + j takes query tiles
  // n_ptiles - 1 - j and j of head group r (a long and a short item, the
  // same amount of work in every workgroup; the pairs in flight share the
  // K/V of a few heads)
  // With a head count that is a multiple of 8 the order is also XCD-aware:
  // workgroups are dealt to the 8 XCDs in turn (w mod 8), so head r goes to
  // XCD r mod 8 and each XCD takes its heads one after another, keeping a
  // head's K/V in one L2.
  const int hp = (p.n_ptiles + 1) / 2;
  const bool xcd = per_ptile % 8 == 0;
  const int wx = xcd ? (wg & 7) : 0, wi = xcd ? wg >> 3 : wg;  // XCD, index on it
  const int per_head = PAIR ? hp : p.n_ptiles;
  const int pr = xcd ? (wi / per_head) * 8 + wx : wi / per_head;  // head group
  const int pj = wi % per_head;                                    // pair / query tile of it
  const int n_my = PAIR ? (p.n_ptiles - 1 - pj > pj ? 2 : 1) : 1;
  const int half_items = (n_items + 1) / 2;
  const int item0 = (CAUSAL && !PAIR && wg >= half_items) ? n_items - 1 - (wg - half_items) : wg;

  // RoPE frequencies (the two-part split of each of the D/2 angles): the
  // 4-wave kernel keeps a copy in LDS that every wave writes itself (the
  // same values, read back only by the wave that wrote them), so a rotation
  // reads them with a few LDS loads instead of holding 64 registers through
  // the key loop; the 8-wave kernel reads them from the parameters per item.
  constexpr bool RQ_LDS = RQ && HALVES == 1;
  if constexpr (RQ_LDS) {
    if (lane < D / 2) {
      rtab[lane] = p.rope_fhi[lane];
      rtab[D / 2 + lane] = p.rope_flo[lane];
    }
  }

#pragma unroll 1
  for (int itn = 0; itn < n_my; ++itn) {
    // every wave is done with the previous item's LDS stages before any
    // wave's loads for this item may land in them
    if (itn > 0) asm volatile("s_barrier" ::: "memory");
    // unpaired causal items: longest first (query tiles from the last one
    // down, all heads of a tile together); non-causal ones are all equally
    // long and go head-major like the pairs (pr, pj above), so the
    // workgroups in flight share the K/V of a few heads (with all heads in
    // flight at once, the K/V of a long sequence outgrows the caches)
    const int ptile = PAIR ? (itn == 0 ? p.n_ptiles - 1 - pj : pj) : CAUSAL ? p.n_ptiles - 1 - item0 / per_ptile : pj;
    int rest = (PAIR || !CAUSAL) ? pr : item0 % per_ptile;
    const int hg = rest % p.n_hgroups;
    rest /= p.n_hgroups;
    const int kvh = rest % p.Hkv;
    const int b = rest / p.Hkv;
    const int head = kvh * p.G + hg * p.GP + (wq % p.GP);
    const int p0 = ptile * p.P;
    const int pw0 = p0 + (wq / p.GP) * 32;
    const int qpos = pw0 + m;
    const int kend = CAUSAL ? min(p.S, p0 + p.P) : p.S;
    const int n_kt = (kend + BN - 1) / BN;  // key tiles the workgroup streams
    // local tile i of this half is key tile HALVES i + half; both halves run
    // n_loc iterations (a half's last tile may lie past the end: fully masked)
    const int n_loc = (n_kt + HALVES - 1) / HALVES;
    auto tl = [&](int i) { return HALVES * i + half; };
    // key tiles this wave computes (a prefix of them; wave-uniform)
    const int n_w = pw0 >= p.S ? 0 : CAUSAL ? min(n_kt, min(pw0 + 31, p.S - 1) / BN + 1) : n_kt;

    const size_t kv_row0 = ((size_t)b * p.Hkv + kvh) * p.S;
    const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.k) + kv_row0 * ROWB;
    const uint8_t* vg = reinterpret_cast<const uint8_t*>(p.v) + kv_row0 * ROWB;
    // DMA of this wave's rows of key tile t; the buffer range ends at the
    // end of the sequence, so rows past it (and tiles past the end) read as
    // zero without a memory access.  Every tile index issues the same number
    // of loads, which keeps the vmcnt arithmetic below exact.
    auto tile_rsrc = [&](const uint8_t* src, int t) {
      const int key0 = t * BN;
      const int range = max(0, p.S - key0) * ROWB;
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src + (size_t)min(key0, p.S) * ROWB), (short)0,
                                               range, kBufferRsrcWord3);
    };
    // this wave's first row of a stage, made opaque by the caller once per
    // group of loads, so the compiler forms each load's LDS address with one
    // scalar add instead of keeping all of them
    auto wave_row = [&]() {
      int wrow = hoff + wq * (RPI * IPW * ROWB);
      asm volatile("" : "+s"(wrow));
      return wrow;
    };
    // load u (0..IPW-1) of this wave's share of a tile
    auto dma1 = [&](__amdgpu_buffer_rsrc_t rs, uint8_t* dst, const int* loff, int u, int wrow) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_AS(void, dst + wrow + RPI * u * ROWB), 16, loff[u], 0, 0, 0);
    };
    auto dma = [&](const uint8_t* src, uint8_t* dst, const int* loff, int t) {
      const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src, t);
      const int wrow = wave_row();
#pragma unroll
      for (int u = 0; u < IPW; ++u) dma1(rs, dst, loff, u, wrow);
    };

    // ---- Q fragments (B operand of S^T = K Q^T), rotated (RoPE) and
    //      multiplied by softmax_scale * log2(e), one rounding to the input type ----
    uint32_t qf[NKK * 4];
    {
      // rows past the sequence end (a ragged last tile) read row S - 1
      // instead: their results are never stored, and the loads need no branch
      const int qld = min(qpos, p.S - 1);
      const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + (((size_t)b * p.Hq + head) * p.S + qld) * D;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const u32x4 w = ldg16(qrow + 16 * kk + 8 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[4 * kk + e] = w[e];
      }
    }
    // loads issued after the Q rows: K(0), then one batch per pipeline slot
    // b = -(NS-1) .. -1, each {K(b + NS), V(b + NS - 1)} (see the loop)
    dma(kg, kst(ic<0>{}), dk, tl(0));
    auto prologue_batch = [&](auto bb) {
      constexpr int bi = decltype(bb)::value;  // b + NS - 1, 0 .. NS - 2
      dma(kg, kst(ic<bi + 1>{}), dk, tl(bi + 1));
      dma(vg, vst(ic<bi>{}), dv, tl(bi));
    };
    prologue_batch(ic<0>{});
    if constexpr (NS > 2) {
      prologue_batch(ic<1>{});
      prologue_batch(ic<2>{});
    }
    {
      const float c = p.scale_log2;
      if (RQ) {
        // element j of k-step kk sits at d = 16 kk + 8 hh + j; its rotate-half
        // partner d + D/2 is in k-step kk + NKK/2 of the same lane
#pragma unroll
        for (int kk = 0; kk < NKK / 2; ++kk) {
          float fhk[8], flk[8];  // frequencies of the 8 elements of k-step kk
          if constexpr (RQ_LDS) {
            const f32x4* th = reinterpret_cast<const f32x4*>(rtab + 16 * kk + 8 * hh);
            const f32x4* tlo = reinterpret_cast<const f32x4*>(rtab + D / 2 + 16 * kk + 8 * hh);
            const f32x4 h0 = th[0], h1 = th[1], l0 = tlo[0], l1 = tlo[1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              fhk[j] = h0[j];
              fhk[4 + j] = h1[j];
              flk[j] = l0[j];
              flk[4 + j] = l1[j];
            }
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              fhk[j] = p.rope_fhi[16 * kk + 8 * hh + j];
              flk[j] = p.rope_flo[16 * kk + 8 * hh + j];
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w1 = qf[4 * kk + e], w2 = qf[4 * (kk + NKK / 2) + e];
            float r1[2], r2[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const float fh = fhk[2 * e + s], fl = flk[2 * e + s];
              const float rev = __builtin_amdgcn_fractf((float)qpos * fh) + (float)qpos * fl;
              const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
              const float x1 = Tag::to_f32(s ? (w1 >> 16) : (w1 & 0xffff));
              const float x2 = Tag::to_f32(s ? (w2 >> 16) : (w2 & 0xffff));
              r1[s] = (x1 * cs - x2 * sn) * c;
              r2[s] = (x2 * cs + x1 * sn) * c;
            }
            qf[4 * kk + e] = Tag::pack2(r1[0], r1[1]);
            qf[4 * (kk + NKK / 2) + e] = Tag::pack2(r2[0], r2[1]);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NKK * 4; ++j)
          qf[j] = Tag::pack2(Tag::to_f32(qf[j] & 0xffff) * c, Tag::to_f32(qf[j] >> 16) * c);
      }
    }
    auto qfrag = [&](int kk) { return u32x4{qf[4 * kk], qf[4 * kk + 1], qf[4 * kk + 2], qf[4 * kk + 3]}; };

    // ---- running state ----
    f32x16 acc_o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
    f32x16 sA[NB], sB[NB];  // score tiles of even / odd key tiles (exponent domain, minus the reference)
    f32x16 negm = {};       // -reference of this lane's row, the first S MFMA's accumulator input
    float m_ref = 0.f;      // reference (exponent domain), equal in both lanes of a row
    float l_run = 0.f;      // sum over this lane's keys of the probabilities
    uint32_t pf[CPB][4];    // probabilities of the tile being multiplied into V (B operand)

    auto krd = [&](const uint8_t* kb, int j) {
      return *reinterpret_cast<const u32x4*>(kb + koff[j % NKK] + 32 * (j / NKK) * ROWB);
    };
    auto vrd = [&](const uint8_t* vb, int j) {
      const int db = j / CPB, c = j % CPB;
      const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(v4i16, vb + voff[db] + 16 * c * ROWB));
      const v4i16 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(v4i16, vb + voff[db] + (16 * c + 8) * ROWB));
      const u32x2 a1 = __builtin_bit_cast(u32x2, x1), a2 = __builtin_bit_cast(u32x2, x2);
      return u32x4{a1[0], a1[1], a2[0], a2[1]};
    };
    // tiles crossing the diagonal or the sequence end need the mask: tile t
    // (keys t BN .. t BN + BN - 1) does iff t BN + BN > S or (causal) its last
    // key lies past the wave's first row pw0, i.e. iff t >= t_mask
    const int t_mask = CAUSAL ? min(p.S / BN, (pw0 + 1) / BN) : p.S / BN;
    auto needs_mask = [&](int t) { return t >= t_mask; };
    // mask of key tile t: keys past the causal bound or the sequence -> -inf
    auto mask = [&](f32x16* s, int t) {
      const int lim = (CAUSAL ? min(qpos, p.S - 1) : p.S - 1) - t * BN - 4 * hh;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * nb + 8 * (r >> 2) + (r & 3) > lim) s[nb][r] = kNegInf;
    };
    // exponentials of values v, v+1 of score tile s (v even), and their
    // packing into pf / the row sum: split so that the packing can trail the
    // exponentials by one chunk (no in-order issue stall on the exp results)
    auto expv2 = [&](f32x16* s, int v, float& e0, float& e1) {
      e0 = fast_exp2(s[v / 16][v % 16]);
      e1 = fast_exp2(s[v / 16][v % 16 + 1]);
    };
    auto packv2 = [&](int v, float e0, float e1) {
      const int nb = v / 16, r = v % 16;
      const uint32_t pk = Tag::pack2(e0, e1);
      pf[2 * nb + (r >> 3)][(r & 7) >> 1] = pk;
      if constexpr (ATTN_SP_LSUM == 0) l_run = Tag::sum2(pk, l_run);
      else if constexpr (ATTN_SP_LSUM == 1) l_run = (l_run + Tag::to_f32(pk & 0xffff)) + Tag::to_f32(pk >> 16);
      else l_run = (l_run + e0) + e1;
    };
    auto expv = [&](f32x16* s, int v) {
      float e0, e1;
      expv2(s, v, e0, e1);
      packv2(v, e0, e1);
    };
    // an empty use of the probabilities of k-steps 0 and 1 and of the row
    // sum after the S phase: the exponentials made there then stay in the
    // block of the S MFMAs they are interleaved with (nothing may sink them
    // towards their use after the mask branch)
    auto pin_p = [&]() {
#pragma unroll
      for (int c = 0; c < CPB / 2; ++c)
        asm volatile("" ::"v"(pf[c][0]), "v"(pf[c][1]), "v"(pf[c][2]), "v"(pf[c][3]));
      asm volatile("" ::"v"(l_run));
    };
    auto pfrag = [&](int c) { return u32x4{pf[c][0], pf[c][1], pf[c][2], pf[c][3]}; };
    // The softmax work of a score tile is spread over the 2 x 16 MFMAs of an
    // iteration.  A lane's 32 values form 16 pairs (pair q: values 2q, 2q+1);
    // pairs 0-7 (the keys of PV k-steps 0 and 1) are exponentiated between
    // the S MFMAs of the next tile, pairs 8-15 (k-steps 2 and 3) between the
    // first PV MFMAs, which take k-steps 0 and 1 first (k-step-major order).
    // A pair is packed (rounded to the input type, added to the row sum) one
    // MFMA after its exponentials, so no in-order issue waits for them.  The
    // row maximum of the next tile is spread over all PV MFMAs.  Each MFMA
    // and its share form one chunk fenced by scheduling barriers.
    constexpr int NP = NB * 8;  // pairs per lane
    // S-phase chunk of first-half pair q (0..7)
    auto s_chunk = [](int q) { return q * NJS / (NP / 2); };
    // PV-phase chunk of second-half pair q (8..15): k-step 2 is first used at
    // chunk 2 NDB, k-step 3 at chunk 3 NDB
    auto pv_chunk = [](int q) {
      return q < NP / 2 + 4 ? (q - NP / 2) * (2 * NDB - 1) / 4 : 2 * NDB + (q - NP / 2 - 4) * (NDB - 1) / 4;
    };
    float ex[NP][2];  // exponentials between their chunk and their packing
    // S of the tile in stage ST into s (accumulating onto `base`), with the
    // first half of the exponentials of the previous tile `sp` (if any) and,
    // if `dk_rs`, this iteration's loads (K loads in the first half of the
    // chunks, V loads in the second)
    auto s_phase = [&](auto stc, f32x16* s, const f32x16& base, f32x16* sp, bool loads,
                       __amdgpu_buffer_rsrc_t krs, uint8_t* kdst, __amdgpu_buffer_rsrc_t vrs, uint8_t* vdst) {
      const uint8_t* kb = kst(stc) + hoff;
      const int wrow = loads ? wave_row() : 0;
      constexpr int KPF = ATTN_SP_KPF;  // K fragments read this many MFMAs ahead
      u32x4 fa[KPF + 1];
#pragma unroll
      for (int x = 0; x < KPF; ++x) fa[x] = krd(kb, x);
#pragma unroll
      for (int j = 0; j < NJS; ++j) {
        if (j + KPF < NJS) fa[(j + KPF) % (KPF + 1)] = krd(kb, j + KPF);
        const int kk = j % NKK, nb = j / NKK;
        s[nb] = Tag::mfma32(fa[j % (KPF + 1)], qfrag(kk), kk == 0 ? base : s[nb]);
        if (sp) {
#pragma unroll
          for (int q = 0; q < NP / 2; ++q) {
            if (s_chunk(q) == j) expv2(sp, 2 * q, ex[q][0], ex[q][1]);
            if (s_chunk(q) + 1 == j) packv2(2 * q, ex[q][0], ex[q][1]);
          }
        }
        if (loads) {
#pragma unroll
          for (int u = 0; u < IPW; ++u) {
            if (j == 1 + 2 * u) dma1(krs, kdst, dk, u, wrow);
            if (j == NJS / 2 + 1 + 2 * u) dma1(vrs, vdst, dv, u, wrow);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (sp) {
#pragma unroll
        for (int q = 0; q < NP / 2; ++q)
          if (s_chunk(q) + 1 == NJS) packv2(2 * q, ex[q][0], ex[q][1]);
      }
    };
    // PV of the tile in stage ST (probabilities in pf), k-step-major, with
    // the second half of the exponentials of that tile `sp` (if any) and the
    // row maximum of the next score tile `sn` (if any) between the MFMAs;
    // V^T fragments are read VPF chunks ahead.  Returns the row maximum
    // (both lanes of the pair).
    auto pv_phase = [&](auto stc, f32x16* sp, f32x16* sn) {
      const uint8_t* vb = vst(stc) + hoff;
      constexpr int VPF = ATTN_SP_VPF;  // V^T fragments read this many MFMAs ahead
      auto vix = [](int j) { return (j % NDB) * CPB + j / NDB; };  // chunk j: k-step j / NDB, block j % NDB
      u32x4 fv[VPF + 1];
#pragma unroll
      for (int x = 0; x < VPF; ++x) fv[x] = vrd(vb, vix(x));
      float mx = kNegInf, mx2 = kNegInf;
#pragma unroll
      for (int j = 0; j < NJV; ++j) {
        if (j + VPF < NJV) fv[(j + VPF) % (VPF + 1)] = vrd(vb, vix(j + VPF));
        acc_o[j % NDB] = Tag::mfma32(fv[j % (VPF + 1)], pfrag(j / NDB), acc_o[j % NDB]);
        if (sp) {
#pragma unroll
          for (int q = NP / 2; q < NP; ++q) {
            if (pv_chunk(q) == j) expv2(sp, 2 * q, ex[q][0], ex[q][1]);
            if (pv_chunk(q) + 1 == j) packv2(2 * q, ex[q][0], ex[q][1]);
          }
        }
        if (sn) {
#pragma unroll
          for (int m2 = 0; m2 < NP; ++m2) {  // max3 over pair m2 of the next tile
            if (m2 * NJV / NP == j) {
              const float a = sn[m2 / 8][(2 * m2) % 16], c = sn[m2 / 8][(2 * m2) % 16 + 1];
              if (m2 & 1) mx2 = fmaxf(mx2, fmaxf(a, c));
              else mx = fmaxf(mx, fmaxf(a, c));
            }
          }
          // opaque per chunk: the max chain is not regrouped into one tree
          // at the end of the block, away from the MFMAs it overlaps
          asm volatile("" : "+v"(mx), "+v"(mx2));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return pair_max32(fmaxf(mx, mx2));
    };
    // move the reference of rows whose tile maximum (relative, `mx`) is above
    // it: O, l and the pending score tile `s` are rescaled (wave-uniform branch)
    auto rescale = [&](f32x16* s, float mx) {
      if (__ballot(mx > kLazy)) {
        const float d = fmaxf(mx, 0.f);
        const float alpha = fast_exp2(-d);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[nb] -= d;
        m_ref += d;
#pragma unroll
        for (int r = 0; r < 16; ++r) negm[r] = -m_ref;
      }
    };

    // ---- prologue: S of tile 0 and the initial reference ----
    constexpr bool PP = HALVES == 2 && ATTN_SP_PINGPONG;
    if (PP && half == 1) asm volatile("s_barrier" ::: "memory");  // the second half runs one barrier behind
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * IPW * (NS - 1)));  // K(0) of this wave landed
    asm volatile("s_barrier" ::: "memory");                      // ... and of every wave
    {
      const f32x16 zero = {};
      s_phase(ic<0>{}, sA, zero, nullptr, false, tile_rsrc(kg, 0), nullptr, tile_rsrc(vg, 0), nullptr);
      if (needs_mask(tl(0))) mask(sA, tl(0));
      float mx = kNegInf;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sA[nb][r]);
      mx = pair_max32(mx);
      m_ref = mx == kNegInf ? 0.f : mx;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sA[nb] -= m_ref;
#pragma unroll
      for (int r = 0; r < 16; ++r) negm[r] = -m_ref;
    }

    // ---- key loop over the n_kt tiles of the workgroup.  Iteration i: wait
    // for K(i+1) and V(i) (the batch issued NS - 1 iterations earlier) and
    // the barrier; issue batch i = {K(i + NS) into the stage of K(i),
    // V(i + NS - 1) into the stage of V(i - 1)}, both read by every wave
    // before this barrier; then
    //   S(i+1) MFMAs || exponentials of S(i)  ->  P(i)
    //   mask S(i+1)
    //   PV(i) MFMAs  || row maximum of S(i+1)
    //   rescale if a row's maximum grew by more than 2^8.
    // Every iteration has the same straight-line body: a wave whose causal
    // bound ends before the workgroup's last tile computes fully masked tiles
    // there (probabilities exactly 0), and the S of the tile after the last
    // one (read from a stage the loads filled with zeros) is never used. ----
    auto iter = [&](auto phc, int i) {
      constexpr int PH = decltype(phc)::value;  // i % NS
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * IPW * (NS - 2)));
      asm volatile("s_barrier" ::: "memory");
      f32x16* sc = (PH & 1) ? sB : sA;  // S(i)
      f32x16* sn = (PH & 1) ? sA : sB;  // S(i+1)
      // loads of this iteration: K(i + NS) into the stage of K(i), V(i + NS - 1)
      // into the stage of V(i - 1), spread over the S MFMAs
      s_phase(ic<PH + 1>{}, sn, negm, sc, true, tile_rsrc(kg, tl(i + NS)), kst(ic<PH>{}), tile_rsrc(vg, tl(i + NS - 1)),
              vst(ic<PH + NS - 1>{}));
      pin_p();
      if constexpr (PP) asm volatile("s_barrier" ::: "memory");
      if (needs_mask(tl(i + 1))) mask(sn, tl(i + 1));
      const float mx = pv_phase(ic<PH>{}, sc, sn);
      rescale(sn, mx);
    };
#pragma unroll 1
    for (int i0 = 0; i0 < n_loc; i0 += NS) {
      iter(ic<0>{}, i0);
      if (i0 + 1 >= n_loc) break;
      iter(ic<1>{}, i0 + 1);
      if constexpr (NS > 2) {
        if (i0 + 2 >= n_loc) break;
        iter(ic<2>{}, i0 + 2);
        if (i0 + 3 >= n_loc) break;
        iter(ic<3>{}, i0 + 3);
      }
    }

    // ---- epilogue: (8 waves) the second half hands its O, reference and
    // row sum to the first through LDS (the stage arrays, free once every
    // wave is past its key loop and its loads have landed), then O / l is
    // stored.  A half that saw no key of a row (row sum 0) has no reference
    // for it and gets weight 0. ----
    if (PP && half == 0) asm volatile("s_barrier" ::: "memory");  // (the first half catches up)
    float l = pair_sum32(l_run);  // row sum (both lanes of the row)
    float f0 = 1.f, f1 = 0.f;
    float* xch = nullptr;
    if constexpr (HALVES == 2) {
      // wave wq of either half: one exchange area of (NDB * 16 + 2) x 64 floats
      uint8_t* area = wq == 0 ? k0 : wq == 1 ? k1 : wq == 2 ? v0 : v1;
      xch = reinterpret_cast<float*>(area);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's loads into the stages have landed
      asm volatile("s_barrier" ::: "memory");
      if (half == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) xch[(db * 16 + r) * 64 + lane] = acc_o[db][r];
        xch[(NDB * 16) * 64 + lane] = m_ref;
        xch[(NDB * 16 + 1) * 64 + lane] = l;
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the LDS stores are done
      asm volatile("s_barrier" ::: "memory");
      if (half == 0) {
        const float l1 = xch[(NDB * 16 + 1) * 64 + lane];
        const float m0 = l > 0.f ? m_ref : kNegInf;
        const float m1 = l1 > 0.f ? xch[(NDB * 16) * 64 + lane] : kNegInf;
        const float M = fmaxf(m0, m1);
        f0 = m0 == kNegInf ? 0.f : fast_exp2(m0 - M);
        f1 = m1 == kNegInf ? 0.f : fast_exp2(m1 - M);
        l = l * f0 + l1 * f1;
        m_ref = M;
      }
    }
    const float inv = l > 0.f ? p.out_scale / l : 0.f;
    if constexpr (HALVES == 1) {
      // O / l leaves through LDS, so that every global store writes 16-byte
      // pieces of whole rows (a lane's accumulator holds 4-element pieces of
      // one row: stored directly, each store instruction would touch 32 rows).
      // Wave wq transposes through stage array wq once every wave is past its
      // key loop and its loads into the stages have landed; the barrier at the
      // start of the next item keeps that item's loads out until all waves
      // have read their rows back.
      uint8_t* area = wq == 0 ? k0 : wq == 1 ? k1 : wq == 2 ? v0 : v1;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      asm volatile("s_barrier" ::: "memory");
      if (n_w > 0) {
        // lane indices made opaque here: the addresses derived from them are
        // then formed in the epilogue, not hoisted out of the item loop (where
        // they would hold registers through the whole key loop)
        int lm = m, ln = lane;
        asm volatile("" : "+v"(lm), "+v"(ln));
        auto stage_out = [&](auto odt) {
          constexpr int OD = decltype(odt)::value;
          constexpr int ES = OD == ATTN_F32 ? 4 : 2;  // bytes per output element
          constexpr int RB = D * ES;                  // bytes per output row
          constexpr int CPR = RB / 16;                // 16-byte pieces per row (XOR-swizzled by row)
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
          // all reads first, then all stores; the buffer range ends at the
          // sequence end, so rows past it are dropped without a branch
          uint8_t* obase = reinterpret_cast<uint8_t*>(p.o) + (((size_t)b * p.Hq + head) * p.S + pw0) * RB;
          const __amdgpu_buffer_rsrc_t ors =
              __builtin_amdgcn_make_buffer_rsrc(obase, (short)0, max(0, min(p.S - pw0, 32)) * RB, kBufferRsrcWord3);
          u32x4 ov[32 / RPR];
#pragma unroll
          for (int i = 0; i < 32 / RPR; ++i) {
            const int r = RPR * i + ln / CPR, c = ln % CPR;
            ov[i] = *reinterpret_cast<const u32x4*>(area + r * RB + 16 * (c ^ (r % CPR)));
          }
#pragma unroll
          for (int i = 0; i < 32 / RPR; ++i)
            __builtin_amdgcn_raw_buffer_store_b128(ov[i], ors, (RPR * i + ln / CPR) * RB + 16 * (ln % CPR), 0, ATTN_SP_OAUX);
        };
        if (p.out_dtype == ATTN_BF16) stage_out(ic<ATTN_BF16>{});
        else if (p.out_dtype == ATTN_F16) stage_out(ic<ATTN_F16>{});
        else stage_out(ic<ATTN_F32>{});
        if (p.lse && hh == 0 && qpos < p.S)
          p.lse[((size_t)b * p.Hq + head) * p.S + qpos] = l > 0.f ? (m_ref + __log2f(l)) * kLn2 : kNegInf;
      }
    } else if (half == 0 && qpos < p.S && n_w > 0) {
      const size_t row = ((size_t)b * p.Hq + head) * p.S + qpos;
      // one branch on the output type for the whole row, not one per store
      auto store_row = [&](auto odt) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float o4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * g4 + e;
              o4[e] = (acc_o[db][r] * f0 + xch[(db * 16 + r) * 64 + lane] * f1) * inv;
            }
            store4(p.o, row * D + 32 * db + 8 * g4 + 4 * hh, decltype(odt)::value, o4[0], o4[1], o4[2], o4[3]);
          }
      };
      if (p.out_dtype == ATTN_BF16) store_row(ic<ATTN_BF16>{});
      else if (p.out_dtype == ATTN_F16) store_row(ic<ATTN_F16>{});
      else store_row(ic<ATTN_F32>{});
      if (p.lse && hh == 0) p.lse[row] = l > 0.f ? (m_ref + __log2f(l)) * kLn2 : kNegInf;
    }
  }
}

template <class Tag, int D, bool CAUSAL, bool RQ>
static void launch_sp_t(const PrefillParams& p, int halves, hipStream_t st) {
  const long long heads = (long long)p.B * p.Hkv * p.n_hgroups;
  const unsigned grid = (unsigned)(CAUSAL && ATTN_SP_PAIR ? (p.n_ptiles + 1) / 2 * heads : p.n_ptiles * heads);
  if (halves == 2)
    hipLaunchKernelGGL((prefill_sp_kernel<Tag, D, CAUSAL, RQ, ATTN_SP_STAGES, 2>), dim3(grid), dim3(512), 0, st, p);
  else
    hipLaunchKernelGGL((prefill_sp_kernel<Tag, D, CAUSAL, RQ, ATTN_SP_STAGES, 1>), dim3(grid), dim3(256), 0, st, p);
}

template <class Tag, int D>
static void launch_sp_d(const PrefillParams& p, bool causal, bool rq, int halves, hipStream_t st) {
  if (causal) {
    if (rq) launch_sp_t<Tag, D, true, true>(p, halves, st);
    else launch_sp_t<Tag, D, true, false>(p, halves, st);
  } else {
    if (rq) launch_sp_t<Tag, D, false, true>(p, halves, st);
    else launch_sp_t<Tag, D, false, false>(p, halves, st);
  }
}

void launch_prefill_sp(const PrefillParams& p, bool bf16, bool causal, bool rope_q, int halves, hipStream_t st) {
  const int D = p.D;
  if (bf16) {
    if (D == 64) launch_sp_d<Bf16Tag, 64>(p, causal, rope_q, halves, st);
    else launch_sp_d<Bf16Tag, 128>(p, causal, rope_q, halves, st);
  } else {
    if (D == 64) launch_sp_d<F16Tag, 64>(p, causal, rope_q, halves, st);
    else launch_sp_d<F16Tag, 128>(p, causal, rope_q, halves, st);
  }
}

}  // namespace attn
