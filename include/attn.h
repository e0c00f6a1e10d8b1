/*
 * attn.h - C ABI of libattn.so: fused scaled-dot-product attention on MI355X (gfx950).
 *
 * The operation (per batch b, query i, query head h):
 *
 *     x_j  = scale * <q_i, k_j>                  raw dot product, scaled afterwards
 *     x_j  = softcap * tanh(x_j / softcap)       only when softcap != 0
 *     x_j += slope_h * mask[i, j]                only with an additive mask (attn_prefill_fwd_ex)
 *     keys excluded by the mask are dropped
 *     o_i  = sum_j e^{x_j} v_j / (sum_j e^{x_j} + e^{sink_h})     (sink term only with sinks)
 *
 * computed tile by tile with a running max and running sum, so no score matrix
 * is ever written to memory. Sources: the fa.metal tensor kernel on the
 * "ggml-metal: FA tensor path: gate to the (256, 256) shape" page (score step:
 * scale, softcap, mask; online softmax; final block "sinks, O /= S" with a
 * zero-sum row written as 0; GQA head map h / (Hq / Hkv)); the "UMMA FMHA"
 * page, "Key lessons learned" (the matrix product is unscaled, the scale is
 * applied afterwards); the "MLA Decode Attention Kernel API Reference" page,
 * Background and parameters (rows gathered from a paged cache by a row list,
 * causal mask from each key's absolute position against the token's).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; inputs are
 *     read only. The library never allocates, frees or synchronises on the
 *     call path: it validates on the host, enqueues kernels on `stream` and
 *     returns. Outputs are valid once the stream has executed the work.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   - bf16 tensors are IEEE bfloat16 bit patterns; fp32 is IEEE binary32;
 *     fp16 is IEEE binary16.
 *   - Operand types (the _ex entry point and attn_decode_fwd): K and V are
 *     bf16 or fp16 (kv_dtype); Q is bf16, fp16 or fp32 (q_dtype) and is
 *     rounded (nearest even) to the K/V type on load, since both products run
 *     on 16-bit MFMAs with fp32 accumulation (the fa.metal tensor kernel on the
 *     "ggml-metal: FA tensor path" page takes fp16 K/V with an fp32 Q). The
 *     probabilities feed the second product in the K/V type as well.
 *   - All argument checks run before any HIP call. On an error status nothing
 *     has been enqueued and the outputs are untouched (ATTN_ERR_HIP: a launch
 *     failed; outputs are then undefined). attn_last_error() gives a message.
 *   - Thread-safe; the library holds no state across calls, apart from the
 *     per-GPU scratch of attn_decode_fwd_noalloc (see there).
 *   - GQA: query head h reads KV head h / (Hq / Hkv) (contiguous groups);
 *     Hq must be a multiple of Hkv.
 *   - Causal masking is bottom-right aligned: query i of a sequence with Sq
 *     queries and Sk keys sits at absolute position Sk - Sq + i and sees keys
 *     j <= Sk - Sq + i. A row that sees no key (and has no sink) is written
 *     as 0 with lse = -inf; with a sink but no key it is 0 as well.
 *   - sinks (optional, NULL = none): fp32 [Hq], one raw logit per query head,
 *     not scaled and not softcapped; it joins the softmax denominator and adds
 *     nothing to the numerator.
 *   - Supported (dk, dv): (16,16) (32,32) (64,64) (96,96) (128,128) (192,192)
 *     (256,256) (192,128) for prefill and paged decode; (576,512) for gathered
 *     decode. Other legal pairs return ATTN_ERR_UNSUPPORTED.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 4

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1,   /* NULL required pointer, non-positive size, Hq % Hkv != 0, ... */
    ATTN_ERR_UNSUPPORTED = 2,   /* legal but not built: (dk, dv) pair, mode combination, sizes past a launch limit */
    ATTN_ERR_HIP = 3            /* a HIP launch failed */
} attn_status;

typedef enum attn_dtype {
    ATTN_BF16 = 0,
    ATTN_F32 = 1,
    ATTN_F16 = 2     /* IEEE binary16 */
} attn_dtype;

/* ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

/* Static description of a status code. */
const char* attn_status_string(int status);

/* Message of the last failed call on this thread ("" if none). */
const char* attn_last_error(void);

/*
 * Prefill (dense) attention: the fa.metal tensor kernel of the "ggml-metal: FA tensor
 * path: gate to the (256, 256) shape" page for a whole query block at once (its score
 * step, online softmax, final "sinks, O /= S" block and GQA head map), with the scale
 * applied to the unscaled product as on the "UMMA FMHA" page, "Key lessons learned".
 *   q     bf16 [B, Sq, Hq, dk]   contiguous
 *   k     bf16 [B, Sk, Hkv, dk]  contiguous
 *   v     bf16 [B, Sk, Hkv, dv]  contiguous
 *   o     [B, Sq, Hq, dv] contiguous, element type o_dtype (ATTN_BF16 or ATTN_F32);
 *         bf16 results are rounded to nearest even from the fp32 result.
 *   lse   optional fp32 [B, Hq, Sq] (NULL = not written): natural-log
 *         log-sum-exp of the row's live scores and sink (-inf if none).
 *   scale multiplies the raw dot product (typically 1/sqrt(dk)); must be finite and > 0.
 *   causal 0/1; softcap >= 0 (0 = off); sinks optional fp32 [Hq].
 * Accumulation is fp32; the probabilities feed the second product as bf16.
 * Launch-size limits (ATTN_ERR_UNSUPPORTED past them): K and V of one batch
 * entry each under 4 GiB; B * Hq * (ceil(Sq / 128) + 1) * 256 under 2^32.
 */
attn_status attn_prefill_fwd(const void* q, const void* k, const void* v,
                             void* o, int o_dtype, float* lse,
                             int B, int Hq, int Hkv, int Sq, int Sk, int dk, int dv,
                             float scale, int causal, float softcap, const float* sinks,
                             void* stream);

/*
 * General prefill: operand types, an additive mask and ALiBi slopes (the
 * mask and max_bias arguments of the fa.metal tensor kernel on the
 * "ggml-metal: FA tensor path" page: the mask entry, times the head's slope,
 * is added to the score after the softcap). Arguments as attn_prefill_fwd, plus:
 *   q_dtype  ATTN_BF16, ATTN_F16 or ATTN_F32 (q is then [B, Sq, Hq, dk] of that type)
 *   kv_dtype ATTN_BF16 or ATTN_F16 (k and v of that type)
 *   mask  IEEE fp16 [mask_batch, mask_heads, Sq, mask_row_stride], contiguous,
 *         16-byte aligned; entry [b % mask_batch, h % mask_heads, i, j] is added
 *         for query i, key j of batch b and query head h (columns j >= Sk are
 *         ignored). -inf drops the key. NULL = no mask (max_bias then has
 *         nothing to scale).
 *   mask_batch, mask_heads >= 1 (1 = shared by all batch entries / heads).
 *   mask_row_stride >= Sk, a multiple of 4 (elements between query rows);
 *         one [Sq, mask_row_stride] slab must be under 4 GiB.
 *   max_bias >= 0: ALiBi. Head h's slope is m0^(h+1) for h < n, else
 *         m1^(2(h - n) + 1), with n the largest power of two <= Hq,
 *         m0 = 2^(-max_bias / n), m1 = 2^(-max_bias / (2n)); 0 gives slope 1.
 * causal may be combined with the mask (both apply). attn_prefill_fwd is this
 * call with bf16 Q, K, V and no mask.
 */
attn_status attn_prefill_fwd_ex(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                                void* o, int o_dtype, float* lse,
                                int B, int Hq, int Hkv, int Sq, int Sk, int dk, int dv,
                                float scale, int causal, float softcap, const float* sinks,
                                const void* mask, int mask_batch, int mask_heads,
                                int64_t mask_row_stride, float max_bias,
                                void* stream);

/*
 * Workspace (bytes) that attn_decode_fwd needs for these sizes: the split-KV
 * partial results (paged: fp32 output rows; gathered: bf16 output rows divided
 * by their own sum; plus the running max and sum per row and split).
 * Sk_max is the largest sequence length (paged mode) or n_sel (gathered mode).
 * Returns 0 for sizes that attn_decode_fwd would reject in either mode (invalid,
 * or past the mode-independent launch-size limits below).
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk_max, int dk, int dv);

/*
 * Decode attention: Sq query rows per sequence (Sq = 1 is the single-token
 * case) against a KV cache read in one of two modes. Paged mode is the same
 * operation as the prefill (same page and steps) over keys addressed through a
 * block table; gathered mode follows the "MLA Decode Attention Kernel API
 * Reference" page, Background and parameters (rows gathered from the cache by a
 * row list in its native layout, a key live iff its position is at or before the
 * token's, the token's own row as one more key) and its Notes (the tokens of a
 * call batched into the matrix products). The keys are split into
 * fixed-size ranges processed in parallel, then merged by log-sum-exp. The
 * range length depends only on the sizes passed here and to
 * attn_decode_workspace_bytes: gathered 64..1024 keys; paged 256..4096 keys, or,
 * for Sk_max >= 16384 at head dims up to 128, the shortest power of two up to
 * 1024 or multiple of 1024 keys whose expected number of non-empty ranges
 * (lengths taken spread up to Sk_max) fills the GPU's wave slots about once. Launch-size limits
 * (ATTN_ERR_UNSUPPORTED past them): B and the number of ranges at most 65535
 * each; B * Sq * Hq under 2^26 output rows; paged mode
 * Hkv * ceil(Sq * (Hq / Hkv) / 16) under 2^26; gathered mode
 * B * ceil(Hq / 64) * ranges under 2^31.
 *
 *   q   [B, Sq, Hq, dk] contiguous, of type q_dtype (bf16, fp16 or fp32);
 *   caches of type kv_dtype (bf16 or fp16);   o [B, Sq, Hq, dv] of type o_dtype.
 *
 * Paged mode (block_table != NULL, row_index == NULL):
 *   k_cache [n_blocks, Hkv, block_size, dk], v_cache [n_blocks, Hkv, block_size, dv]
 *   block_table int32 [B, max_blocks_per_seq]: logical key j of sequence b is
 *     slot j % block_size of physical block block_table[b, j / block_size];
 *   seq_lens int32 [B] on the device, each in [0, Sk_max]; sequence b has keys
 *     [0, seq_lens[b]). block_size must be 16, 32, 64 or 128 (multiple of 16).
 *   Any Sq: query columns (Sq * Hq / Hkv per KV head, e.g. several tokens of a
 *     speculative draft) are processed in groups of 32.
 *   The caller guarantees table entries for j < seq_lens[b] are valid blocks.
 *
 * Gathered mode (row_index != NULL, block_table == NULL): Hkv must be 1 and Sq 1.
 *   k_cache, v_cache row arrays with a common row stride kv_row_stride
 *     (elements, multiple of 8): the key of row r is k_cache[r*stride .. +dk),
 *     its value v_cache[r*stride .. +dv) (v_cache may alias k_cache, e.g. the
 *     value being the row's first dv columns).
 *   row_index int32 [B, n_sel]: the rows token b attends to (each valid);
 *   key_pos  fp32  [B, n_sel]: absolute position of each selected key;
 *   q_pos    int32 [B]: position of token b. With causal, key j is live iff
 *     key_pos[b, j] <= q_pos[b]; without causal every selected key is live.
 *   Sk_max must equal n_sel.
 *   k_cur, v_cur (optional, both or neither): rows [B, kv_row_stride] of kv_dtype
 *     holding token b's own key (first dk columns of k_cur row b) and value
 *     (first dv of v_cur row b); they join the selected rows as one more key at
 *     position q_pos[b], always live (the page's n_keys = n_prior + 1 with
 *     kv_row_cur). With v_cache == k_cache, v_cur must equal k_cur. NULL in
 *     paged mode.
 *
 *   workspace: device buffer of at least attn_decode_workspace_bytes(...) bytes,
 *     16-byte aligned, owned by the caller; contents on entry do not matter.
 *   Two calls that share a workspace must be ordered on one stream.
 */
attn_status attn_decode_fwd(const void* q, const void* k_cache, const void* v_cache,
                            void* o, int o_dtype, int q_dtype, int kv_dtype,
                            int B, int Hq, int Hkv, int Sq, int Sk_max, int dk, int dv,
                            float scale, int causal, float softcap, const float* sinks,
                            const int32_t* block_table, int block_size, int max_blocks_per_seq,
                            const int32_t* seq_lens,
                            const int32_t* row_index, const float* key_pos, const int32_t* q_pos,
                            int n_sel, int64_t kv_row_stride,
                            const void* k_cur, const void* v_cur,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Decode without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments, modes, results and errors are those of attn_decode_fwd; the split-KV partial
 * results go to a static device array of the library (ATTN_NOALLOC_SCRATCH_BYTES per GPU,
 * held until the process ends) instead of a caller-owned workspace. The call allocates
 * nothing: its first call on a GPU looks up that GPU's copy of the array (the GPU that runs
 * `stream`) and caches the address.
 *   - Sizes whose workspace (attn_decode_workspace_bytes) exceeds ATTN_NOALLOC_SCRATCH_BYTES
 *     return ATTN_ERR_UNSUPPORTED; use attn_decode_fwd with a workspace for them.
 *   - Every call on one GPU shares that GPU's array: two calls whose execution overlaps on
 *     one GPU (different streams, or host threads enqueueing concurrently on different
 *     streams) race and give undefined results. Calls ordered on one stream are safe.
 *   - The array keeps the last call's contents; no call relies on them.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
attn_status attn_decode_fwd_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    void* o, int o_dtype, int q_dtype, int kv_dtype,
                                    int B, int Hq, int Hkv, int Sq, int Sk_max, int dk, int dv,
                                    float scale, int causal, float softcap, const float* sinks,
                                    const int32_t* block_table, int block_size, int max_blocks_per_seq,
                                    const int32_t* seq_lens,
                                    const int32_t* row_index, const float* key_pos, const int32_t* q_pos,
                                    int n_sel, int64_t kv_row_stride,
                                    const void* k_cur, const void* v_cur,
                                    void* stream);

/*
 * Block formats of a quantized KV cache (32 values per block, IEEE fp16
 * scale d first, blocks packed back to back with no padding).
 */
typedef enum attn_qfmt {
    ATTN_Q8_0 = 0,   /* 34-byte blocks: d, 32 x int8 q; value = d * q */
    ATTN_Q4_0 = 1    /* 18-byte blocks: d, 16 bytes; byte j holds q_j (low nibble) and
                        q_{j+16} (high nibble); value = d * (q - 8) */
} attn_qfmt;

/*
 * Dequantize n_blocks blocks of format fmt at src into IEEE fp16 dst
 * [n_blocks * 32] (values in block order): the pre-pass the "ggml-metal: FA
 * tensor path" page runs so that quantized K/V feed the fp16 kernels (then
 * call the attention entry points with kv_dtype = ATTN_F16). d * q is exact in
 * fp32 and rounded once to fp16 (nearest even). src and dst are device
 * buffers, 16-byte aligned, not overlapping; n_blocks = 0 does nothing.
 * Four threads expand one block (8 values each): n_blocks above 2^30 - 64 (a
 * grid of 2^32 threads) gives ATTN_ERR_UNSUPPORTED.
 */
attn_status attn_dequant_fp16(const void* src, int fmt, void* dst, int64_t n_blocks, void* stream);

/*
 * MLA decode tail: the out-absorb and the o-projection that follow MLA decode
 * attention ("MLA Decode Attention Kernel API Reference" page: Background, the
 * out_absorb_w and o_proj_w parameters, Notes: both are batched across the
 * tokens). With K = H * DV:
 *   u[t, h*DV + v] = sum_c w_absorb[h, v, c] * o_lat[t, h, c]   (fp32, rounded to bf16)
 *   y[t, n]        = sum_k u[t, k] * w_o[k, n]                   (fp32 accumulation)
 *   o_lat     bf16 [T, H, R]   the latent attention output (attn_decode_fwd's
 *                              gathered-mode o with dv = R and o_dtype ATTN_BF16)
 *   w_absorb  bf16 [H, DV, R]  each head's value half of the KV up-projection
 *   w_o       bf16 [K, N]      the o-projection, rows head-major (row h*DV + v)
 *   y         [T, N] contiguous, element type y_dtype (ATTN_BF16 or ATTN_F32);
 *             bf16 results are rounded to nearest even from the fp32 sum.
 * Requirements: T, H >= 1; R a multiple of 128; DV a multiple of 16; K a
 * multiple of 128; N a multiple of 128 (at most 128 * 65535); T * N at most
 * 2^34 - 256 (the final sum runs one thread per 4 outputs); every pointer
 * 16-byte aligned; workspace (device, caller-owned, at least
 * attn_mla_tail_workspace_bytes(T, H, R, DV, N) bytes, 16-byte aligned) holds u
 * and the fp32 partial sums of the K slices; it is fully overwritten. The
 * K slices are added in a fixed order, so results are run-to-run identical.
 * All buffers are device memory and must not overlap. Errors:
 * ATTN_ERR_INVALID_ARG for NULL or misaligned pointers, sizes that break the
 * rules above, or a workspace that is too small; nothing is launched then.
 */
size_t attn_mla_tail_workspace_bytes(int T, int H, int R, int DV, int N);
attn_status attn_mla_tail(const void* o_lat, const void* w_absorb, const void* w_o, void* y, int y_dtype,
                          int T, int H, int R, int DV, int N,
                          void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
