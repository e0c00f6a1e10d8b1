// C ABI of libattn.so: argument validation on the host, then kernel launches.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing; see include/attn.h for the contract of each entry point.
#include "attn.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "attn_launch.hpp"

static_assert(attn::kNoallocScratchBytes == ATTN_NOALLOC_SCRATCH_BYTES, "scratch size of the header and the library");

namespace {

thread_local char g_last_error[512] = "";

attn_status fail(attn_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

attn_status ok() {
    g_last_error[0] = '\0';
    return ATTN_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

attn_status check_common(int B, int Hq, int Hkv, int Sq, int dk, int dv, float scale, float softcap,
                         int o_dtype) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || dk <= 0 || dv <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d Sq=%d dk=%d dv=%d)", B, Hq,
                    Hkv, Sq, dk, dv);
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (!(std::isfinite(scale) && scale > 0.f))
        return fail(ATTN_ERR_INVALID_ARG, "scale must be finite and positive");
    if (!(std::isfinite(softcap) && softcap >= 0.f))
        return fail(ATTN_ERR_INVALID_ARG, "softcap must be finite and >= 0 (0 = off)");
    if (o_dtype != ATTN_BF16 && o_dtype != ATTN_F32)
        return fail(ATTN_ERR_INVALID_ARG, "o_dtype must be ATTN_BF16 or ATTN_F32");
    return ATTN_OK;
}

attn_status check_dtypes(int q_dtype, int kv_dtype) {
    if (q_dtype != ATTN_BF16 && q_dtype != ATTN_F32 && q_dtype != ATTN_F16)
        return fail(ATTN_ERR_INVALID_ARG, "q_dtype must be ATTN_BF16, ATTN_F32 or ATTN_F16");
    if (kv_dtype != ATTN_BF16 && kv_dtype != ATTN_F16)
        return fail(ATTN_ERR_INVALID_ARG, "kv_dtype must be ATTN_BF16 or ATTN_F16");
    return ATTN_OK;
}

// Launch-size limits of a decode call that hold in both modes: B and the key-split count
// are grid dimensions of the split kernels (at most 65535 each), and the combine runs one
// 64-thread workgroup per output row in a grid dimension of fewer than 2^32 threads. Within
// them the workspace size cannot overflow. Returns nullptr when the shape fits.
const char* decode_too_large(int B, const attn::DecodePlan& pl) {
    if (B > 65535 || pl.n_split > 65535) return "B and the key-split count must each be at most 65535";
    if (pl.n_rows > (int64_t(1) << 26) - 1) return "B * Sq * Hq must be under 2^26 output rows";
    return nullptr;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_INVALID_ARG: return "invalid argument";
        case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
        case ATTN_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

const char* attn_last_error(void) { return g_last_error; }

static attn_status prefill_impl(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype, void* o,
                                int o_dtype, float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int dk, int dv,
                                float scale, int causal, float softcap, const float* sinks, const void* mask,
                                int mask_batch, int mask_heads, int64_t mask_row_stride, float max_bias,
                                void* stream) {
    if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o are required");
    attn_status st = check_common(B, Hq, Hkv, Sq, dk, dv, scale, softcap, o_dtype);
    if (st != ATTN_OK) return st;
    st = check_dtypes(q_dtype, kv_dtype);
    if (st != ATTN_OK) return st;
    if (Sk <= 0) return fail(ATTN_ERR_INVALID_ARG, "Sk must be positive (got %d)", Sk);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    if (mask != nullptr) {
        if (mask_batch <= 0 || mask_heads <= 0)
            return fail(ATTN_ERR_INVALID_ARG, "mask_batch and mask_heads must be positive");
        if (mask_row_stride < Sk || mask_row_stride % 4 != 0)
            return fail(ATTN_ERR_INVALID_ARG, "mask_row_stride must be >= Sk and a multiple of 4 (got %lld)",
                        (long long)mask_row_stride);
        if (!aligned16(mask)) return fail(ATTN_ERR_INVALID_ARG, "mask must be 16-byte aligned");
        if ((double)Sq * (double)mask_row_stride * 2.0 >= 4294967296.0)
            return fail(ATTN_ERR_UNSUPPORTED, "one (batch, head) mask slab must be under 4 GiB");
    }
    if (!(std::isfinite(max_bias) && max_bias >= 0.f))
        return fail(ATTN_ERR_INVALID_ARG, "max_bias must be finite and >= 0");
    if (!attn::prefill_supported(dk, dv))
        return fail(ATTN_ERR_UNSUPPORTED, "prefill (dk, dv) = (%d, %d) is not built", dk, dv);
    // one workgroup of 64 * NW threads per 32 * NW query rows (NW = 4 or 8) of one (head, batch
    // entry): the 1-D grid holds at most (ceil(Sq / 128) + 1) * 256 threads per (head, batch
    // entry), and a grid dimension holds fewer than 2^32 threads
    if ((double)B * Hq * ((Sq + 127) / 128 + 1) * 256.0 > 4294967295.0)
        return fail(ATTN_ERR_UNSUPPORTED, "problem too large for one launch (B * Hq * Sq too large)");
    if ((double)Sk * Hkv * (dk > dv ? dk : dv) * 2.0 >= 4294967296.0)
        return fail(ATTN_ERR_UNSUPPORTED, "K or V of one batch entry must be under 4 GiB");

    attn::PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.sinks = sinks;
    a.o_f32 = o_dtype == ATTN_F32;
    a.q_type = q_dtype;
    a.kv_f16 = kv_dtype == ATTN_F16;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Sq = Sq;
    a.Sk = Sk;
    a.dk = dk;
    a.dv = dv;
    a.scale = scale;
    a.causal = causal ? 1 : 0;
    a.softcap = softcap;
    a.mask = mask;
    a.mask_stride = (long long)mask_row_stride;
    a.mask_batch = mask ? mask_batch : 1;
    a.mask_heads = mask ? mask_heads : 1;
    a.max_bias = max_bias;
    hipError_t e = attn::launch_prefill(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
    return ok();
}

attn_status attn_prefill_fwd(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse,
                             int B, int Hq, int Hkv, int Sq, int Sk, int dk, int dv, float scale, int causal,
                             float softcap, const float* sinks, void* stream) {
    return prefill_impl(q, ATTN_BF16, k, v, ATTN_BF16, o, o_dtype, lse, B, Hq, Hkv, Sq, Sk, dk, dv, scale, causal,
                        softcap, sinks, nullptr, 1, 1, 0, 0.f, stream);
}

attn_status attn_prefill_fwd_ex(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype, void* o,
                                int o_dtype, float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int dk, int dv,
                                float scale, int causal, float softcap, const float* sinks, const void* mask,
                                int mask_batch, int mask_heads, int64_t mask_row_stride, float max_bias,
                                void* stream) {
    return prefill_impl(q, q_dtype, k, v, kv_dtype, o, o_dtype, lse, B, Hq, Hkv, Sq, Sk, dk, dv, scale, causal,
                        softcap, sinks, mask, mask_batch, mask_heads, mask_row_stride, max_bias, stream);
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk_max, int dk, int dv) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Sk_max < 0 || dk <= 0 || dv <= 0 || Hq % Hkv != 0) return 0;
    const attn::DecodePlan pl = attn::decode_plan(B, Hq, Hkv, Sq, Sk_max, dk, dv);
    return decode_too_large(B, pl) ? 0 : pl.ws_bytes;
}

// Checks and launches a decode call. noalloc: the split-KV workspace is the library's static
// device scratch (workspace / workspace_bytes are ignored) instead of the caller's buffer.
static attn_status decode_impl(const void* q, const void* k_cache, const void* v_cache, void* o, int o_dtype,
                               int q_dtype, int kv_dtype, int B,
                               int Hq, int Hkv, int Sq, int Sk_max, int dk, int dv, float scale, int causal,
                               float softcap, const float* sinks, const int32_t* block_table, int block_size,
                               int max_blocks_per_seq, const int32_t* seq_lens, const int32_t* row_index,
                               const float* key_pos, const int32_t* q_pos, int n_sel, int64_t kv_row_stride,
                               const void* k_cur, const void* v_cur, void* workspace, size_t workspace_bytes,
                               bool noalloc, void* stream) {
    if (!q || !k_cache || !v_cache || !o) return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache and o are required");
    attn_status st = check_common(B, Hq, Hkv, Sq, dk, dv, scale, softcap, o_dtype);
    if (st != ATTN_OK) return st;
    st = check_dtypes(q_dtype, kv_dtype);
    if (st != ATTN_OK) return st;
    const bool paged = block_table != nullptr;
    const bool gathered = row_index != nullptr;
    if (paged == gathered)
        return fail(ATTN_ERR_INVALID_ARG, "exactly one of block_table (paged) and row_index (gathered) must be given");
    if (Sk_max < 0) return fail(ATTN_ERR_INVALID_ARG, "Sk_max must be >= 0");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
        return fail(ATTN_ERR_INVALID_ARG, "q, caches and o must be 16-byte aligned");
    if (paged) {
        if (!seq_lens) return fail(ATTN_ERR_INVALID_ARG, "paged mode needs seq_lens");
        if (block_size != 16 && block_size != 32 && block_size != 64 && block_size != 128)
            return fail(ATTN_ERR_INVALID_ARG, "block_size must be 16, 32, 64 or 128 (got %d)", block_size);
        if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * block_size < Sk_max)
            return fail(ATTN_ERR_INVALID_ARG, "max_blocks_per_seq * block_size must cover Sk_max");
        if ((int64_t)Sq * (Hq / Hkv) > (1 << 20))
            return fail(ATTN_ERR_UNSUPPORTED, "paged decode needs Sq * (Hq / Hkv) <= 2^20");
        if (k_cur || v_cur) return fail(ATTN_ERR_INVALID_ARG, "k_cur / v_cur apply to gathered mode only");
    } else {
        if (!key_pos || !q_pos) return fail(ATTN_ERR_INVALID_ARG, "gathered mode needs key_pos and q_pos");
        if (Hkv != 1 || Sq != 1) return fail(ATTN_ERR_INVALID_ARG, "gathered mode needs Hkv == 1 and Sq == 1");
        if (n_sel <= 0 || n_sel != Sk_max) return fail(ATTN_ERR_INVALID_ARG, "gathered mode needs n_sel == Sk_max > 0");
        if (kv_row_stride < dk || kv_row_stride < dv || kv_row_stride % 8 != 0)
            return fail(ATTN_ERR_INVALID_ARG, "kv_row_stride must be a multiple of 8 and >= dk, dv");
        if ((k_cur == nullptr) != (v_cur == nullptr))
            return fail(ATTN_ERR_INVALID_ARG, "k_cur and v_cur go together");
        if (k_cur && (!aligned16(k_cur) || !aligned16(v_cur)))
            return fail(ATTN_ERR_INVALID_ARG, "k_cur and v_cur must be 16-byte aligned");
        if (k_cur && v_cache == k_cache && v_cur != k_cur)
            return fail(ATTN_ERR_INVALID_ARG, "v_cache == k_cache needs v_cur == k_cur (value = key-row prefix)");
    }
    if (!attn::decode_supported(dk, dv, gathered))
        return fail(ATTN_ERR_UNSUPPORTED, "%s decode (dk, dv) = (%d, %d) is not built", gathered ? "gathered" : "paged",
                    dk, dv);
    const attn::DecodePlan pl = attn::decode_plan(B, Hq, Hkv, Sq, Sk_max, dk, dv);
    if (const char* why = decode_too_large(B, pl))
        return fail(ATTN_ERR_UNSUPPORTED, "decode grid too large (B = %d, Hq = %d, Sq = %d, %d key splits): %s", B, Hq,
                    Sq, pl.n_split, why);
    // the paged kernel's first grid dimension holds Hkv * (16-column query groups at most) wavefronts,
    // the gathered kernel's second one the 64-head groups
    if (paged && (int64_t)Hkv * (((int64_t)Sq * (Hq / Hkv) + 15) / 16) > (int64_t(1) << 26) - 1)
        return fail(ATTN_ERR_UNSUPPORTED, "decode grid too large: Hkv * Sq * (Hq / Hkv) / 16 must be under 2^26");
    // the gathered split pass runs one workgroup per (token, 64 query heads, key range) in a
    // 1-D grid
    if (gathered && (long long)B * attn::gathered_head_groups(Hq) * pl.n_split > 0x7fffffffLL)
        return fail(ATTN_ERR_UNSUPPORTED, "decode grid too large: B * ceil(Hq / 64) * key ranges must be under 2^31");
    if (noalloc) {
        if (pl.ws_bytes > attn::kNoallocScratchBytes)
            return fail(ATTN_ERR_UNSUPPORTED,
                        "attn_decode_fwd_noalloc: these sizes need %zu bytes of split-KV scratch, more than the "
                        "%zu-byte static scratch; use attn_decode_fwd with a workspace",
                        pl.ws_bytes, attn::kNoallocScratchBytes);
        // all argument checks are done: the first HIP call is the scratch lookup
        hipError_t e = attn::noalloc_scratch((hipStream_t)stream, &workspace);
        if (e != hipSuccess)
            return fail(ATTN_ERR_HIP, "no-allocation scratch lookup failed: %s", hipGetErrorString(e));
    } else {
        if (!workspace || workspace_bytes < pl.ws_bytes)
            return fail(ATTN_ERR_INVALID_ARG, "workspace of %zu bytes needed (got %zu)", pl.ws_bytes, workspace_bytes);
        if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    }

    attn::DecodeArgs a;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.o = o;
    a.sinks = sinks;
    a.o_f32 = o_dtype == ATTN_F32;
    a.q_type = q_dtype;
    a.kv_f16 = kv_dtype == ATTN_F16;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Sq = Sq;
    a.Sk_max = Sk_max;
    a.dk = dk;
    a.dv = dv;
    a.scale = scale;
    a.causal = causal ? 1 : 0;
    a.softcap = softcap;
    a.block_table = block_table;
    a.block_size = block_size;
    a.max_blocks = max_blocks_per_seq;
    a.seq_lens = seq_lens;
    a.row_index = row_index;
    a.key_pos = key_pos;
    a.q_pos = q_pos;
    a.n_sel = n_sel;
    a.row_stride = kv_row_stride;
    a.k_cur = k_cur;
    a.v_cur = v_cur;
    a.workspace = workspace;
    hipError_t e = attn::launch_decode(a, pl, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    return ok();
}

attn_status attn_decode_fwd(const void* q, const void* k_cache, const void* v_cache, void* o, int o_dtype,
                            int q_dtype, int kv_dtype, int B,
                            int Hq, int Hkv, int Sq, int Sk_max, int dk, int dv, float scale, int causal,
                            float softcap, const float* sinks, const int32_t* block_table, int block_size,
                            int max_blocks_per_seq, const int32_t* seq_lens, const int32_t* row_index,
                            const float* key_pos, const int32_t* q_pos, int n_sel, int64_t kv_row_stride,
                            const void* k_cur, const void* v_cur, void* workspace, size_t workspace_bytes,
                            void* stream) {
    return decode_impl(q, k_cache, v_cache, o, o_dtype, q_dtype, kv_dtype, B, Hq, Hkv, Sq, Sk_max, dk, dv, scale,
                       causal, softcap, sinks, block_table, block_size, max_blocks_per_seq, seq_lens, row_index,
                       key_pos, q_pos, n_sel, kv_row_stride, k_cur, v_cur, workspace, workspace_bytes, false, stream);
}

attn_status attn_decode_fwd_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, int o_dtype,
                                    int q_dtype, int kv_dtype, int B,
                                    int Hq, int Hkv, int Sq, int Sk_max, int dk, int dv, float scale, int causal,
                                    float softcap, const float* sinks, const int32_t* block_table, int block_size,
                                    int max_blocks_per_seq, const int32_t* seq_lens, const int32_t* row_index,
                                    const float* key_pos, const int32_t* q_pos, int n_sel, int64_t kv_row_stride,
                                    const void* k_cur, const void* v_cur, void* stream) {
    return decode_impl(q, k_cache, v_cache, o, o_dtype, q_dtype, kv_dtype, B, Hq, Hkv, Sq, Sk_max, dk, dv, scale,
                       causal, softcap, sinks, block_table, block_size, max_blocks_per_seq, seq_lens, row_index,
                       key_pos, q_pos, n_sel, kv_row_stride, k_cur, v_cur, nullptr, 0, true, stream);
}

attn_status attn_dequant_fp16(const void* src, int fmt, void* dst, int64_t n_blocks, void* stream) {
    if (fmt != ATTN_Q8_0 && fmt != ATTN_Q4_0) return fail(ATTN_ERR_INVALID_ARG, "fmt must be ATTN_Q8_0 or ATTN_Q4_0");
    if (n_blocks < 0) return fail(ATTN_ERR_INVALID_ARG, "n_blocks must be >= 0");
    if (n_blocks == 0) return ok();
    if (!src || !dst) return fail(ATTN_ERR_INVALID_ARG, "src and dst are required");
    if (!aligned16(src) || !aligned16(dst)) return fail(ATTN_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
    // four threads per block in a 1-D grid of fewer than 2^32 threads (64 blocks per workgroup)
    if (n_blocks > ((int64_t)1 << 30) - 64)
        return fail(ATTN_ERR_UNSUPPORTED, "n_blocks above 2^30 - 64: too many blocks for one launch");
    hipError_t e = attn::launch_dequant(src, fmt, dst, (long long)n_blocks, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "dequant launch failed: %s", hipGetErrorString(e));
    return ok();
}

size_t attn_mla_tail_workspace_bytes(int T, int H, int R, int DV, int N) {
    if (T <= 0 || H <= 0 || R <= 0 || DV <= 0 || N <= 0) return 0;
    return attn::tail_plan(T, H, R, DV, N).ws_bytes;
}

attn_status attn_mla_tail(const void* o_lat, const void* w_absorb, const void* w_o, void* y, int y_dtype, int T,
                          int H, int R, int DV, int N, void* workspace, size_t workspace_bytes, void* stream) {
    if (!o_lat || !w_absorb || !w_o || !y || !workspace)
        return fail(ATTN_ERR_INVALID_ARG, "o_lat, w_absorb, w_o, y and workspace are required");
    if (T <= 0 || H <= 0 || R <= 0 || DV <= 0 || N <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (T=%d H=%d R=%d DV=%d N=%d)", T, H, R, DV, N);
    if (y_dtype != ATTN_BF16 && y_dtype != ATTN_F32)
        return fail(ATTN_ERR_INVALID_ARG, "y_dtype must be ATTN_BF16 or ATTN_F32");
    if (R % 128 != 0) return fail(ATTN_ERR_INVALID_ARG, "R (%d) must be a multiple of 128", R);
    if (DV % 16 != 0) return fail(ATTN_ERR_INVALID_ARG, "DV (%d) must be a multiple of 16", DV);
    const long long K = (long long)H * DV;
    if (K % 128 != 0) return fail(ATTN_ERR_INVALID_ARG, "H * DV (%lld) must be a multiple of 128", K);
    if (N % 128 != 0) return fail(ATTN_ERR_INVALID_ARG, "N (%d) must be a multiple of 128", N);
    if (N / 128 > 65535) return fail(ATTN_ERR_INVALID_ARG, "N (%d) exceeds 128 * 65535", N);
    // the slice sum runs one thread per 4 outputs in a 1-D grid of fewer than 2^32 threads
    if ((long long)T * N > (1LL << 34) - 256)
        return fail(ATTN_ERR_INVALID_ARG, "T * N (%lld) exceeds 2^34 - 256", (long long)T * N);
    if (K > INT32_MAX / 2 || (long long)H * (DV / 16) > INT32_MAX)
        return fail(ATTN_ERR_INVALID_ARG, "H * DV (%lld) too large", K);
    if (!aligned16(o_lat) || !aligned16(w_absorb) || !aligned16(w_o) || !aligned16(y) || !aligned16(workspace))
        return fail(ATTN_ERR_INVALID_ARG, "o_lat, w_absorb, w_o, y and workspace must be 16-byte aligned");
    const attn::TailPlan pl = attn::tail_plan(T, H, R, DV, N);
    if (workspace_bytes < pl.ws_bytes)
        return fail(ATTN_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
                    pl.ws_bytes);
    attn::TailArgs a;
    a.o_lat = o_lat;
    a.w_absorb = w_absorb;
    a.w_o = w_o;
    a.y = y;
    a.y_f32 = y_dtype == ATTN_F32;
    a.T = T;
    a.H = H;
    a.R = R;
    a.DV = DV;
    a.N = N;
    a.workspace = workspace;
    hipError_t e = attn::launch_mla_tail(a, pl, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "MLA tail launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
