/*
 * attn.h - C ABI of the MI355X (gfx950) attention forward library.
 *
 * Scaled-dot-product attention forward with online softmax: causal GQA
 * prefill with fused RoPE, split-context GQA decode against a static KV
 * cache, absorbed-MLA decode over a 448-d latent plus 64-d RoPE cache, and
 * the split-softmax combine step that both decode paths end with.
 *
 * Conventions shared by every call:
 *  - All tensor pointers are DEVICE pointers to contiguous row-major arrays
 *    with the head dimension innermost.  The caller owns every buffer,
 *    including the workspace; the library allocates and frees nothing and
 *    keeps no mutable global state, so calls are thread-safe.  The one
 *    exception is attn_decode_gqa_noalloc, whose partials live in a static
 *    device array shared by all its calls on a GPU (see there).
 *  - Calls only enqueue kernels on `stream` and return; nothing synchronises
 *    with the host, so every call is legal inside hipGraph stream capture.
 *  - Host-side argument checks run before anything is launched; on a
 *    non-OK status nothing was enqueued.  A failed kernel launch returns
 *    ATTN_ERR_LAUNCH.  Values that live in device memory (kv_len) cannot be
 *    checked on the host: they are clamped to [0, cap] on the device, and a
 *    sequence with kv_len == 0 gets an all-zero output row.
 *  - Tensor pointers must be 16-byte aligned (lse pointers 4-byte aligned).
 *  - softmax_scale multiplies q.k before the softmax (the caller passes
 *    1/sqrt(head_dim) for the usual scaling).
 *
 * Sources (pages cited by title and section):
 *  - "Lesson: shape adaptive attention negative 20260722", rows "What was
 *    tried" and "Conditions": causal GQA prefill/decode with RoPE fused into
 *    attention, one global tile configuration, eager vs graph replay.
 *  - "Fixed-budget decode audit", sections "Which implementation was
 *    tested" and "Setup and interpretation": split-context decode (split
 *    128) against a static append cache (capacity 2056 for context 2048),
 *    MLA with a 448-d latent + 64-d RoPE per token; section "A: group-entry
 *    queries and one joint history scan": the softmax-part merge.
 *  - Persistent-attention digest (hada.io), benchmark section: Z=4, H=32
 *    forward in fp16 and fp8 e5m2 ("float8e5").
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL                    */
    ATTN_ERR_SHAPE = 2,       /* a size is <= 0, inconsistent or too large     */
    ATTN_ERR_DTYPE = 3,       /* unknown dtype or unsupported dtype combination */
    ATTN_ERR_ALIGN = 4,       /* a pointer is not suitably aligned             */
    ATTN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required       */
    ATTN_ERR_UNSUPPORTED = 6, /* valid request the library does not implement  */
    ATTN_ERR_LAUNCH = 7       /* the HIP runtime rejected a kernel launch      */
} attn_status;

typedef enum attn_dtype {
    ATTN_F32 = 0,
    ATTN_F16 = 1,
    ATTN_BF16 = 2,
    ATTN_FP8_E5M2 = 3         /* OCP E5M2 bytes (1 sign, 5 exponent, 2 mantissa) */
} attn_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* attn_status_str(attn_status s);

/* ------------------------------------------------------------------------ *
 * Prefill: O = softmax(scale * rope(Q) rope(K)^T [+ causal mask]) V
 *
 * Operation: for query head h of sequence b, KV head g = h / (Hq/Hkv); with
 * RoPE, rows of Q and K at position p are rotated in rotate-half pairs
 * (i, i + D/2) by angle p * rope_theta^(-2i/D), positions 0..S-1; causal
 * means key j is visible to query i iff j <= i.
 *
 *   q    [B, Hq,  S, D]  in_dtype
 *   k, v [B, Hkv, S, D]  in_dtype
 *   o    [B, Hq,  S, D]  out_dtype
 *   lse  [B, Hq,  S]     float32, natural-log log-sum-exp of the scaled
 *                        scores of each row; may be NULL (not written).
 *
 * in_dtype: ATTN_F32, ATTN_F16, ATTN_BF16 or ATTN_FP8_E5M2.
 * out_dtype: ATTN_F32, ATTN_F16 or ATTN_BF16.  D: 64 or 128.
 * rope_theta <= 0 disables RoPE (RoPE with fp8 input, or with S > 65536:
 * ATTN_ERR_UNSUPPORTED).  softmax_scale * q_descale * k_descale must be a
 * positive finite number (ATTN_ERR_SHAPE otherwise).
 * q_descale, k_descale multiply the scores and v_descale the output (per-
 * tensor dequantisation factors; pass 1.0 for unscaled inputs).
 * Math is fp32 with fp32 accumulation; 16-bit and fp8 inputs use MFMA.
 *
 * attn_prefill_gqa_rope rotates Q and K inside the attention kernel: each Q
 * row once, each K tile while it is staged, i.e. once for every query tile
 * that reads it.  One kernel on `stream`, no workspace.
 *
 * attn_prefill_gqa_rope_ws is the same operation with RoPE on K done once
 * per key: a first kernel writes the rotated K to the caller's workspace
 * (attn_prefill_gqa_rope_workspace_bytes() bytes, 16-byte aligned, not
 * overlapping any other argument; contents on entry are ignored and on
 * return hold the rotated K), then the attention kernel reads K from there
 * and rotates only its Q rows.  Rotated values are rounded to in_dtype in
 * both forms, so the two give the same result up to the angle's last
 * bits.  The workspace size is B*Hkv*S*D*2 bytes for 16-bit inputs with
 * rope_theta > 0 and 0 otherwise (then `workspace` may be NULL and only the
 * attention kernel runs).  ATTN_ERR_WORKSPACE if it is needed and missing
 * or too small.  Two kernels on `stream` (one without RoPE).
 * ------------------------------------------------------------------------ */
attn_status attn_prefill_gqa_rope(const void* q, const void* k, const void* v, void* o,
                                  float* lse, int B, int Hq, int Hkv, int S, int D,
                                  attn_dtype in_dtype, attn_dtype out_dtype,
                                  float softmax_scale, int causal, float rope_theta,
                                  float q_descale, float k_descale, float v_descale,
                                  hipStream_t stream);
size_t attn_prefill_gqa_rope_workspace_bytes(int B, int Hkv, int S, int D, attn_dtype in_dtype,
                                             float rope_theta);
attn_status attn_prefill_gqa_rope_ws(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int B, int Hq, int Hkv, int S, int D,
                                     attn_dtype in_dtype, attn_dtype out_dtype,
                                     float softmax_scale, int causal, float rope_theta,
                                     float q_descale, float k_descale, float v_descale,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Tile-configuration sweep: the same prefill with an explicit configuration
 * id in [0, attn_prefill_num_configs()).  Configuration 0 is the one global
 * configuration attn_prefill_gqa_rope and attn_prefill_gqa_rope_ws use; the
 * others exist so that a per-shape sweep can measure how far the global
 * choice is from the best configuration of each shape (the shape-adaptive
 * attention lesson page, row "Actual result": the global candidate's gap to
 * the per-invocation oracle).  For the 16-bit MFMA kernel: 0 = 4-wave
 * workgroups of 128 query rows, one workgroup per work item; 1 = 8-wave
 * workgroups whose halves split the key tiles of 128 rows; 2 = the tiling
 * of 0, software-pipelined (S of the next key tile issued during the softmax
 * of this one); 3 = the kernel of 0 with persistent scheduling when the work
 * items exceed two residency rounds (two resident workgroups per compute
 * unit loop over the items, snake order over the longest-first list), and
 * launched as 0 otherwise; 4 = the kernel of 0 with 32-key tiles (half the
 * LDS, three workgroups per compute unit; RoPE with K rotated per staged
 * tile runs as 0); 5 = the workgroups of 1 with their halves run half a key
 * tile apart, so that one half's softmax overlaps the other half's MFMAs
 * (RoPE with K rotated per staged tile runs as 1); 6 = the kernel of 0 with
 * the K and V tiles staged through registers instead of LDS DMA (RoPE with K
 * rotated per staged tile runs as 0).
 * fp8 inputs: 1 = P in f16 with V upcast; every other id = P rounded to e4m3
 * for the PV MFMA (fp8 x bf8, twice the f16 rate).  fp32 inputs ignore the
 * id (one configuration).  An id out of range returns ATTN_ERR_UNSUPPORTED.
 * With a NULL workspace K is rotated inside the kernel as in
 * attn_prefill_gqa_rope; with a workspace, once per key first, as in
 * attn_prefill_gqa_rope_ws.  ATTN_CONFIG_K_ROTATED or-ed into the id says
 * that the workspace already holds this K rotated (left there by an earlier
 * call with the same k, rope_theta and shapes): the rotation kernel is
 * skipped and only the attention kernel runs, which times it on its own and
 * lets calls that share K reuse the rotation (NULL workspace with the flag:
 * ATTN_ERR_WORKSPACE; without RoPE, or for fp32 and fp8 inputs, the flag
 * changes nothing). */
#define ATTN_CONFIG_K_ROTATED 0x100
int attn_prefill_num_configs(void);
attn_status attn_prefill_gqa_rope_with_config(const void* q, const void* k, const void* v, void* o,
                                              float* lse, int B, int Hq, int Hkv, int S, int D,
                                              attn_dtype in_dtype, attn_dtype out_dtype,
                                              float softmax_scale, int causal, float rope_theta,
                                              float q_descale, float k_descale, float v_descale,
                                              int config, void* workspace, size_t workspace_bytes,
                                              hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Standalone RoPE rotation (the unfused form of the prefill's RoPE step; the
 * shape-adaptive attention lesson page, rows "What was tried" and "Actual
 * result", compares RoPE fused into attention with separate RoPE kernels).
 *
 *   x, y  [B, H, S, D]  dtype; y may equal x (in place), otherwise the two
 *         must not overlap.
 *
 * Row (b, h, s) is rotated as in attn_prefill_gqa_rope: the rotate-half pair
 * (i, i + D/2) turns by angle s * rope_theta^(-2i/D), positions 0..S-1,
 * computed in fp32 and rounded once to dtype.  Applying it to Q and K and
 * then calling attn_prefill_gqa_rope with rope_theta <= 0 gives the same
 * attention as the fused call (up to rounding order).
 *
 * dtype: ATTN_F32, ATTN_F16 or ATTN_BF16 (ATTN_FP8_E5M2: ATTN_ERR_UNSUPPORTED).
 * D even, at most 256, half rows a whole number of 16-byte chunks (D % 16 == 0
 * for 16-bit types, D % 8 == 0 for fp32); S <= 65536; rope_theta a positive
 * finite number (ATTN_ERR_SHAPE otherwise).  Launches one kernel on `stream`.
 * ------------------------------------------------------------------------ */
attn_status attn_rope_rotate(const void* x, void* y, int B, int H, int S, int D, attn_dtype dtype,
                             float rope_theta, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Split-context GQA decode ("flash-decoding"): one new query token per
 * sequence against a static KV cache.  Defined by "Fixed-budget decode
 * audit": section "Which implementation was tested" (a fused split-score
 * kernel over a static append cache), section "Setup and interpretation"
 * (BF16, context 2048 in a cache of capacity 2056, batches 1 to 128) and
 * section "Optimized full-model results" (split size 128, graph replay).
 *
 *   q        [B, Hq, D]        dtype
 *   k_cache  [B, Hkv, cap, D]  dtype (slot t holds the key of position t)
 *   v_cache  [B, Hkv, cap, D]  dtype
 *   kv_len   [B] int32, DEVICE memory: sequence b attends to slots
 *            0..kv_len[b]-1 of its KV head (the new token's own key and
 *            value are already in the cache); slots >= kv_len[b] are
 *            never read, so they may hold anything, NaN included.
 *   o        [B, Hq, D]        dtype
 *   workspace: device scratch of at least attn_decode_gqa_workspace_bytes()
 *            bytes, 256-byte aligned; contents on entry are ignored.  When
 *            that size is 0 the workspace is not used and may be NULL.
 *
 * The context [0, kv_len[b]) of each KV head is cut into equal runs of
 * 32-slot chunks, one per wave; `split` (<= 0: the library default, 128)
 * is the most slots one wave streams.  The 4 waves of a workgroup merge
 * their softmax parts in LDS; a KV head gets ceil(cap / (4 * split))
 * workgroups, and when there is more than one their parts go to the
 * workspace and a combine step merges them (with one, the output is
 * written directly and a single kernel runs).  dtype: ATTN_BF16 or
 * ATTN_F16.  D: 128.  Hq/Hkv <= 16.  split: a multiple of 32 in
 * [32, 1024].  One or two kernels on `stream`.
 * ------------------------------------------------------------------------ */
size_t attn_decode_gqa_workspace_bytes(int B, int Hq, int cap, int D, int split);
attn_status attn_decode_gqa(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* kv_len, void* o, void* workspace,
                            size_t workspace_bytes, int B, int Hq, int Hkv, int D, int cap,
                            int split, attn_dtype dtype, float softmax_scale,
                            hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * attn_decode_gqa without a workspace, for callers that cannot allocate
 * device memory (code under stream capture that must not call hipMalloc,
 * tight serving loops, harnesses that forbid allocation).  The same
 * operation, arguments, kernels and error checks as attn_decode_gqa; the
 * split partials go to a static device array of the library (8 MiB per GPU,
 * kept until the process ends) instead of a caller workspace.
 *   Limit: attn_decode_gqa_workspace_bytes(B, Hq, cap, D, split) must not
 *   exceed 8 MiB (8388608 bytes), else ATTN_ERR_WORKSPACE and nothing is
 *   launched.  The default split at capacity 2056 (five partial parts of
 *   128 floats per query row) fits up to B * Hq = 3251 rows.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (different streams or host threads) race and must be ordered by the
 *   caller.  The array needs no clearing between calls.
 *   The first call on a GPU looks up the array's address there
 *   (hipGetSymbolAddress; ATTN_ERR_LAUNCH if that fails).  No call
 *   allocates or frees memory.
 * ------------------------------------------------------------------------ */
attn_status attn_decode_gqa_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* kv_len, void* o, int B, int Hq, int Hkv, int D,
                                    int cap, int split, attn_dtype dtype, float softmax_scale,
                                    hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Absorbed-MLA decode: H query heads share one latent cache row per token.
 * Defined by "Fixed-budget decode audit": section "Which implementation was
 * tested" (MLA with absorption, a 448-d latent plus a 64-d RoPE part per
 * token) and section "Like-for-like eager absorption comparison" (the
 * "MLA absorbed" row at batch 128, context 2048).
 *
 *   q        [B, H, d_latent + d_rope]    dtype, the absorbed query
 *            [W_UK q_nope ; q_rope] (latent part first)
 *   kv_cache [B, cap, d_latent + d_rope]  dtype, latent then RoPE part
 *   kv_len   [B] int32, DEVICE memory (as for attn_decode_gqa)
 *   o        [B, H, d_latent]             dtype: softmax(scale q c^T) c_lat
 *   workspace: at least attn_decode_mla_workspace_bytes() bytes.
 *
 * Scores use all d_latent + d_rope dims; values are the latent part of the
 * same rows.  dtype: ATTN_BF16 or ATTN_F16.  d_latent = 448, d_rope = 64,
 * H <= 16.  split <= 0 (the default) cuts [0, kv_len[b]) on the device into
 * n equal runs of 32-slot chunks, n = round(compute units / B) clamped to
 * [1, min(16, ceil(cap / 32))], so one setting serves batch 1 and batch 128;
 * otherwise split is a fixed run length in slots, a multiple of 32 in
 * [32, 2048], with ceil(cap / split) <= 65535 (else ATTN_ERR_SHAPE).
 * Launches two kernels on `stream`.
 * ------------------------------------------------------------------------ */
size_t attn_decode_mla_workspace_bytes(int B, int H, int cap, int d_latent, int split);
attn_status attn_decode_mla(const void* q, const void* kv_cache, const int32_t* kv_len,
                            void* o, void* workspace, size_t workspace_bytes, int B, int H,
                            int d_latent, int d_rope, int cap, int split, attn_dtype dtype,
                            float softmax_scale, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Split-softmax combine (the merge of softmax parts).  Defined by
 * "Fixed-budget decode audit", section "A: group-entry queries and one
 * joint history scan" (an output and its log-sum-exp merged with a second
 * part through a sigmoid of the log-sum-exp difference), generalised to
 * many parts; section "Measured group-attention times" names the split
 * reduction this step performs.  For each of R rows,
 *   o[r] = sum_s w_s o_part[r, s] / sum_s w_s,  w_s = exp(lse_part[r, s] - max_s lse_part[r, s]).
 * This equals folding the pairwise merge alpha = sigmoid(lse_b - lse_a),
 * o = (1 - alpha) o_a + alpha o_b over the parts.  A part with
 * lse = -inf is empty and contributes nothing; a row whose parts are all
 * empty gets zeros.
 *
 *   o_part   [R, nsplit, D] float32, each part normalised within itself
 *   lse_part [R, nsplit]    float32, natural log
 *   o        [R, D]         out_dtype (ATTN_F32, ATTN_F16 or ATTN_BF16)
 * D: 1..1024.  The decode calls run this step themselves; it is exported so
 * that it can be called and tested on its own.
 * ------------------------------------------------------------------------ */
attn_status attn_combine_splits(const float* o_part, const float* lse_part, void* o, int R,
                                int nsplit, int D, attn_dtype out_dtype, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Decode neighbours: the steps on either side of decode attention in a
 * session with a static append cache ("Fixed-budget decode audit", section
 * "Setup and interpretation": the cache is appended in place, prompts are
 * prefilled in chunks of 32).
 *
 * attn_kv_append writes T new tokens per sequence into the caches:
 *   k_new, v_new [B, Hkv, T, D]   dtype
 *   q            [B, Hq, T, D]    dtype, nullable: the same tokens' queries,
 *                                 rotated in place when RoPE is on
 *   k_cache, v_cache [B, Hkv, cap, D]  dtype, written at slots
 *                                 L .. L+T-1 with L = kv_len[b]
 *   kv_len       [B] int32 device memory; read on the device (clamped to
 *                [0, cap]); when `advance` is nonzero it becomes
 *                min(L + T, cap) after the append.
 * The slot index is the token's position: K (and q) are rotated as in
 * attn_prefill_gqa_rope at position L + t when rope_theta > 0; V is copied;
 * rope_theta <= 0 copies K too.  Tokens whose slot would be >= cap are not
 * written (precondition: kv_len[b] + T <= cap).  Slots outside the appended
 * range are not touched.  k_new/v_new must not overlap the caches.
 * dtype: ATTN_F32, ATTN_F16 or ATTN_BF16; D even, at most 256, half rows a
 * whole number of 16-byte chunks; with RoPE cap <= 65536.  One kernel (a
 * second, tiny one advances kv_len when a sequence's tokens are shared by
 * several workgroups), enqueued on `stream` (graph-capturable: the lengths
 * live on the device, so replays keep appending).
 *
 * attn_prefill_chunk attends a chunk of T query rows per sequence to the
 * cache prefix:
 *   q       [B, Hq, T, D]      dtype; with rope_theta > 0 the kernel rotates
 *           row t to its position (below) as in attn_prefill_gqa_rope, in
 *           registers (q itself is not written); with rope_theta <= 0 q is
 *           used as given (e.g. already rotated by attn_kv_append)
 *   k_cache, v_cache [B, Hkv, cap, D]  dtype (K already rotated)
 *   kv_len  [B] int32 device memory: key count INCLUDING the chunk's own
 *           tokens (clamped to [0, cap])
 *   o       [B, Hq, T, D]      out_dtype; lse [B, Hq, T] float32 or NULL
 * Row t of sequence b sits at position p = kv_len[b] - T + t and attends to
 * slots 0..p: O = softmax(scale q K^T) V with query head h reading KV head
 * h / (Hq/Hkv).  Rows with p < 0 have no key and get zeros (lse -inf).
 * The key axis is cut into ranges of `split` keys (a multiple of 64; <= 0:
 * a default from the shapes, aiming at ~512 workgroups) that run in
 * parallel; when there is more than one range their partial results go to
 * the caller's workspace (attn_prefill_chunk_workspace_bytes bytes,
 * 256-byte aligned; 0 bytes, workspace may be NULL, when one range covers
 * cap) and the combine kernel merges them.
 * dtype ATTN_BF16 or ATTN_F16 (others: ATTN_ERR_UNSUPPORTED); D 64 or 128;
 * T <= cap; scale a positive finite number; rope_theta not NaN, and with
 * RoPE cap <= 65536 (else ATTN_ERR_UNSUPPORTED); ATTN_ERR_WORKSPACE if the
 * workspace is missing or too small.  One or two kernels on `stream`.
 * ------------------------------------------------------------------------ */
attn_status attn_kv_append(const void* k_new, const void* v_new, void* q, void* k_cache,
                           void* v_cache, int32_t* kv_len, int B, int Hkv, int Hq, int T, int D,
                           int cap, attn_dtype dtype, float rope_theta, int advance,
                           hipStream_t stream);
size_t attn_prefill_chunk_workspace_bytes(int B, int Hq, int Hkv, int T, int D, int cap, int split);
attn_status attn_prefill_chunk(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* kv_len, void* o, float* lse, void* workspace,
                               size_t workspace_bytes, int B, int Hq, int Hkv, int T, int D,
                               int cap, int split, attn_dtype dtype, attn_dtype out_dtype,
                               float softmax_scale, float rope_theta, hipStream_t stream);

/* ------------------------------------------------------------------------
 * One step of chunked prefill into a static append cache, in one call
 * ("Fixed-budget decode audit", "Setup and interpretation": prompts are
 * prefilled chunk by chunk into the static append cache the decode reads):
 * the work of attn_kv_append (advance 0) followed by attn_prefill_chunk, with
 * the cache-length advance carried by the attention's last launch.
 *   q        [B, Hq, T, D]   the chunk's queries, dtype, not rotated (the
 *            attention rotates them in registers when rope_theta > 0)
 *   k_new, v_new [B, Hkv, T, D]  the chunk's keys (not rotated) and values
 *   k_cache, v_cache [B, Hkv, cap, D]  written at slots L_b .. L_b+T-1 (K
 *            rotated to those positions when rope_theta > 0; slots >= cap
 *            are not written)
 *   kv_len   [B] int32 device memory: on entry L_b, the tokens already
 *            cached (EXCLUDING the chunk); on return min(L_b + T, cap)
 *   o, lse, workspace: as attn_prefill_chunk (same workspace size:
 *            attn_prefill_chunk_workspace_bytes)
 * Results equal attn_kv_append(..., advance = 1) followed by
 * attn_prefill_chunk on the same arguments, bit for bit.  For T <= 32 the
 * attention kernel writes the chunk's rows to the cache itself, so the step
 * is two kernels (attention, then the combine, which also advances kv_len;
 * with a single key range the advance is a small kernel of its own); longer
 * chunks are appended by the append kernel first.  Error
 * checks are those of both calls and all run before any work is enqueued,
 * so a rejected call writes nothing; calls sharing kv_len must not overlap.
 * ------------------------------------------------------------------------ */
attn_status attn_prefill_chunk_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                    void* v_cache, int32_t* kv_len, void* o, float* lse, void* workspace,
                                    size_t workspace_bytes, int B, int Hq, int Hkv, int T, int D, int cap,
                                    int split, attn_dtype dtype, attn_dtype out_dtype, float softmax_scale,
                                    float rope_theta, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
