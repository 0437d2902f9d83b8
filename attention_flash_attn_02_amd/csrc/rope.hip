// Standalone rotary position embedding: the unfused form of the prefill's
// RoPE step.  The shape-adaptive attention lesson page (rows "What was tried"
// and "Actual result") compares RoPE fused into the attention kernel with
// RoPE as separate kernels; this kernel rotates Q or K in HBM so that the
// attention kernel can run without RoPE.
//
// Operation (rotate-half): for row (b, h, s) at position s, the pair
// (x[i], x[i + D/2]) becomes (x[i] cos a - x[i+D/2] sin a,
// x[i+D/2] cos a + x[i] sin a) with a = s * theta^(-2i/D), in fp32 with the
// angle reduced to one revolution from an exact three-part split of the
// frequency; the result is rounded once to the element type (round to
// nearest even).
//
// One thread per row and 16-byte chunk of the first half: it loads the
// chunk and its partner chunk D/2 elements later, rotates the pairs and
// stores both, so the rotation is done in place when y == x (every element
// is read and written by the same thread).

#include "common.hpp"
#include "kernels.hpp"
#include "rope_common.hpp"

namespace attn {

struct RopeParams {
  const void* x;
  void* y;
  long long rows;  // B * H * S
  int S, D;
  float rope_fhi[128];
  float rope_fmid[128];
  float rope_flo[128];
};

template <class Tag>
__global__ __launch_bounds__(256) void rope_kernel(const RopeParams p) {
  constexpr int EB = Tag::kBytes;
  constexpr int EPC = 16 / EB;  // elements per 16-byte chunk
  const int half = p.D / 2;
  const int cpr = half / EPC;  // chunks per half row
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= p.rows * cpr) return;
  const long long row = t / cpr;
  const int c = (int)(t % cpr);
  const float pos = (float)(int)(row % p.S);
  const uint8_t* xr = reinterpret_cast<const uint8_t*>(p.x) + row * p.D * EB;
  uint8_t* yr = reinterpret_cast<uint8_t*>(p.y) + row * p.D * EB;
  u32x4 lo = *reinterpret_cast<const u32x4*>(xr + 16 * c);
  u32x4 hi = *reinterpret_cast<const u32x4*>(xr + half * EB + 16 * c);
  rotate_chunk_pair<Tag>(lo, hi, pos, c, p.rope_fhi, p.rope_fmid, p.rope_flo);
  *reinterpret_cast<u32x4*>(yr + 16 * c) = lo;
  *reinterpret_cast<u32x4*>(yr + half * EB + 16 * c) = hi;
}

// ---------------------------------------------------------------------------
// Cache append: the step before decode attention in a static append cache
// ("Fixed-budget decode audit", "Setup and interpretation").  T new tokens
// of sequence b go to slots L .. L+T-1 with L = kv_len[b]; the slot index is
// the token's position, K is rotated to it (rope on), V is copied, and the
// queries of the same tokens are rotated in place at the same positions.
// gridDim.y workgroups per sequence share its rows.  With one workgroup per
// sequence the update kv_len[b] = min(L + T, cap) follows a barrier after
// which every thread has read L; with several, advance_kernel does it as a
// second launch (stream order puts it after every read).
// ---------------------------------------------------------------------------
struct AppendParams {
  const void* k_new;  // [B, Hkv, T, D]
  const void* v_new;  // [B, Hkv, T, D]
  void* q;            // [B, Hq, T, D] rotated in place, or null
  void* k_cache;      // [B, Hkv, cap, D]
  void* v_cache;      // [B, Hkv, cap, D]
  int* kv_len;        // [B]
  int Hkv, Hq, T, D, cap;
  int rope, advance;
  float rope_fhi[128];
  float rope_fmid[128];
  float rope_flo[128];
};

template <class Tag>
__global__ __launch_bounds__(256) void append_kernel(const AppendParams p) {
  constexpr int EB = Tag::kBytes;
  constexpr int EPC = 16 / EB;
  const int b = blockIdx.x;
  const int half = p.D / 2, cpr = half / EPC, cpf = p.D / EPC;  // chunk pairs / chunks per row
  const int L = min(max(p.kv_len[b], 0), p.cap);
  const size_t rowb = (size_t)p.D * EB;
  const int w0 = blockIdx.y * 256 + threadIdx.x, ws = 256 * gridDim.y;
  const uint8_t* kn = reinterpret_cast<const uint8_t*>(p.k_new) + (size_t)b * p.Hkv * p.T * rowb;
  const uint8_t* vn = reinterpret_cast<const uint8_t*>(p.v_new) + (size_t)b * p.Hkv * p.T * rowb;
  uint8_t* kc = reinterpret_cast<uint8_t*>(p.k_cache) + (size_t)b * p.Hkv * p.cap * rowb;
  uint8_t* vc = reinterpret_cast<uint8_t*>(p.v_cache) + (size_t)b * p.Hkv * p.cap * rowb;
  // K: rows (h, t) x chunk pairs
  for (int w = w0; w < p.Hkv * p.T * cpr; w += ws) {
    const int row = w / cpr, c = w % cpr, h = row / p.T, t = row % p.T;
    const int slot = L + t;
    if (slot >= p.cap) continue;
    const uint8_t* src = kn + (size_t)row * rowb;
    uint8_t* dst = kc + ((size_t)h * p.cap + slot) * rowb;
    u32x4 lo = *reinterpret_cast<const u32x4*>(src + 16 * c);
    u32x4 hi = *reinterpret_cast<const u32x4*>(src + half * EB + 16 * c);
    if (p.rope) rotate_chunk_pair<Tag>(lo, hi, (float)slot, c, p.rope_fhi, p.rope_fmid, p.rope_flo);
    *reinterpret_cast<u32x4*>(dst + 16 * c) = lo;
    *reinterpret_cast<u32x4*>(dst + half * EB + 16 * c) = hi;
  }
  // V: rows (h, t) x chunks, copied
  for (int w = w0; w < p.Hkv * p.T * cpf; w += ws) {
    const int row = w / cpf, c = w % cpf, h = row / p.T, t = row % p.T;
    const int slot = L + t;
    if (slot >= p.cap) continue;
    *reinterpret_cast<u32x4*>(vc + ((size_t)h * p.cap + slot) * rowb + 16 * c) =
        *reinterpret_cast<const u32x4*>(vn + (size_t)row * rowb + 16 * c);
  }
  // Q: rows (h, t) x chunk pairs, rotated in place at position L + t
  if (p.q && p.rope) {
    uint8_t* qb = reinterpret_cast<uint8_t*>(p.q) + (size_t)b * p.Hq * p.T * rowb;
    for (int w = w0; w < p.Hq * p.T * cpr; w += ws) {
      const int row = w / cpr, c = w % cpr, t = row % p.T;
      uint8_t* x = qb + (size_t)row * rowb;
      u32x4 lo = *reinterpret_cast<const u32x4*>(x + 16 * c);
      u32x4 hi = *reinterpret_cast<const u32x4*>(x + half * EB + 16 * c);
      rotate_chunk_pair<Tag>(lo, hi, (float)(L + t), c, p.rope_fhi, p.rope_fmid, p.rope_flo);
      *reinterpret_cast<u32x4*>(x + 16 * c) = lo;
      *reinterpret_cast<u32x4*>(x + half * EB + 16 * c) = hi;
    }
  }
  if (p.advance && gridDim.y == 1) {
    __syncthreads();  // every thread has read kv_len[b]
    if (threadIdx.x == 0) p.kv_len[b] = min(L + p.T, p.cap);
  }
}

__global__ __launch_bounds__(256) void advance_kernel(int* kv_len, int B, int T, int cap) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b < B) kv_len[b] = min(max(kv_len[b], 0) + T, cap);
}

void launch_kv_advance(const KvAdvance& adv, hipStream_t stream) {
  hipLaunchKernelGGL(advance_kernel, dim3((unsigned)((adv.B + 255) / 256)), dim3(256), 0, stream, adv.kv_len, adv.B,
                     adv.T, adv.cap);
}

}  // namespace attn

using namespace attn;

extern "C" attn_status attn_rope_rotate(const void* x, void* y, int B, int H, int S, int D, attn_dtype dtype,
                                        float rope_theta, hipStream_t stream) {
  if (!x || !y) return ATTN_ERR_NULL;
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0 || D % 2 != 0) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) {
    if (dtype == ATTN_FP8_E5M2) return ATTN_ERR_UNSUPPORTED;
    return ATTN_ERR_DTYPE;
  }
  if (!(rope_theta > 0.f) || !(rope_theta < 3.0e38f)) return ATTN_ERR_SHAPE;
  const int eb = dtype == ATTN_F32 ? 4 : 2;
  // whole 16-byte chunks in each half row; at most 256 dims
  if (D > 256 || ((D / 2) * eb) % 16 != 0) return ATTN_ERR_UNSUPPORTED;
  if (S > 65536) return ATTN_ERR_UNSUPPORTED;  // exact angle reduction needs pos < 2^16
  if (!attn_host::aligned(x, 16) || !attn_host::aligned(y, 16)) return ATTN_ERR_ALIGN;
  const long long rows = (long long)B * H * S;
  const long long threads = rows * ((D / 2) * eb / 16);
  if ((threads + 255) / 256 > 0x7fffffffLL) return ATTN_ERR_SHAPE;

  RopeParams p{};
  p.x = x; p.y = y; p.rows = rows; p.S = S; p.D = D;
  attn_host::rope_freq_split(rope_theta, D, nullptr, p.rope_fhi, p.rope_flo, p.rope_fmid);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (dtype == ATTN_BF16) hipLaunchKernelGGL((rope_kernel<Bf16Tag>), grid, block, 0, stream, p);
  else if (dtype == ATTN_F16) hipLaunchKernelGGL((rope_kernel<F16Tag>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((rope_kernel<F32Elem>), grid, block, 0, stream, p);
  return attn_host::launch_status();
}

extern "C" attn_status attn_kv_append(const void* k_new, const void* v_new, void* q, void* k_cache,
                                      void* v_cache, int32_t* kv_len, int B, int Hkv, int Hq, int T, int D,
                                      int cap, attn_dtype dtype, float rope_theta, int advance,
                                      hipStream_t stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !kv_len) return ATTN_ERR_NULL;
  if (B <= 0 || Hkv <= 0 || T <= 0 || D <= 0 || cap <= 0 || D % 2 != 0) return ATTN_ERR_SHAPE;
  if (q && Hq <= 0) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) {
    if (dtype == ATTN_FP8_E5M2) return ATTN_ERR_UNSUPPORTED;
    return ATTN_ERR_DTYPE;
  }
  const bool rope = rope_theta > 0.f;
  if (rope_theta != rope_theta || !(rope_theta < 3.0e38f)) return ATTN_ERR_SHAPE;
  const int eb = dtype == ATTN_F32 ? 4 : 2;
  if (D > 256 || ((D / 2) * eb) % 16 != 0) return ATTN_ERR_UNSUPPORTED;
  if (rope && cap > 65536) return ATTN_ERR_UNSUPPORTED;  // exact angle reduction needs pos < 2^16
  if (!attn_host::aligned(k_new, 16) || !attn_host::aligned(v_new, 16) || !attn_host::aligned(k_cache, 16) ||
      !attn_host::aligned(v_cache, 16) || !attn_host::aligned(kv_len, 4) || (q && !attn_host::aligned(q, 16)))
    return ATTN_ERR_ALIGN;
  if ((long long)(Hkv > Hq ? Hkv : Hq) * T * D > (1LL << 30) || (long long)Hkv * cap * D > (1LL << 40))
    return ATTN_ERR_SHAPE;

  AppendParams p{};
  p.k_new = k_new; p.v_new = v_new; p.q = q; p.k_cache = k_cache; p.v_cache = v_cache; p.kv_len = kv_len;
  p.Hkv = Hkv; p.Hq = q ? Hq : 0; p.T = T; p.D = D; p.cap = cap;
  p.rope = rope ? 1 : 0;
  p.advance = advance ? 1 : 0;
  if (rope) attn_host::rope_freq_split(rope_theta, D, nullptr, p.rope_fhi, p.rope_flo, p.rope_fmid);
  // workgroups per sequence: about 256 rotated chunk pairs each (one per thread)
  const long long pairs = (long long)(Hkv + p.Hq) * T * ((D / 2) * eb / 16);
  const long long gy = (pairs + 255) / 256;
  const dim3 grid((unsigned)B, (unsigned)(gy < 1 ? 1 : gy > 1024 ? 1024 : gy)), block(256);
  if (dtype == ATTN_BF16) hipLaunchKernelGGL((append_kernel<Bf16Tag>), grid, block, 0, stream, p);
  else if (dtype == ATTN_F16) hipLaunchKernelGGL((append_kernel<F16Tag>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((append_kernel<F32Elem>), grid, block, 0, stream, p);
  if (advance && grid.y > 1) launch_kv_advance(KvAdvance{kv_len, B, T, cap}, stream);
  return attn_host::launch_status();
}
