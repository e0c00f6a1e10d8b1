// Host-side launch interface between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const float* sinks;
    int o_f32;
    int q_type = 0;  // 0 bf16, 1 fp32, 2 fp16
    int kv_f16 = 0;  // K and V are fp16 (else bf16)
    int B, Hq, Hkv, Sq, Sk, dk, dv;
    float scale;
    int causal;
    float softcap;
    // additive fp16 mask [mask_batch, mask_heads, Sq, mask_stride] (NULL: none) and ALiBi
    const void* mask = nullptr;
    long long mask_stride = 0;
    int mask_batch = 1, mask_heads = 1;
    float max_bias = 0.f;
};

// Returns false if (dk, dv) has no compiled instance.
bool prefill_supported(int dk, int dv);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Head dim (256, 256), built in its own translation unit (called by launch_prefill).
hipError_t launch_prefill_d256(const PrefillArgs& a, hipStream_t stream);

struct DecodeArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    void* o;
    const float* sinks;
    int o_f32;
    int q_type = 0;  // 0 bf16, 1 fp32, 2 fp16
    int kv_f16 = 0;  // K and V are fp16 (else bf16)
    int B, Hq, Hkv, Sq, Sk_max, dk, dv;
    float scale;
    int causal;
    float softcap;
    // paged mode
    const int32_t* block_table;
    int block_size;
    int max_blocks;
    const int32_t* seq_lens;
    // gathered mode
    const int32_t* row_index;
    const float* key_pos;
    const int32_t* q_pos;
    const void* k_cur = nullptr;  // gathered mode: token t's own key / value row (NULL: none)
    const void* v_cur = nullptr;
    int n_sel;
    int64_t row_stride;
    // split-KV scratch
    void* workspace;
};

struct DecodePlan {
    int split_len;   // keys per split (multiple of the kernel's key tile)
    int n_split;     // ceil(Sk_max / split_len)
    int64_t n_rows;  // B * Sq * Hq output rows
    size_t ws_bytes; // partial O (fp32 or bf16, dv per row per split) + (max, sum) per row per split
};

// Size of the static device scratch that attn_decode_fwd_noalloc uses as its workspace.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
// Device address of that scratch on the device that runs `stream` (looked up once per
// device with hipGetSymbolAddress, then cached).
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

bool decode_supported(int dk, int dv, bool gathered);
// Gathered mode: rows per key range the LDS index table holds (a range of up to 1024
// selected keys plus the token's own row, rounded up to whole 32-key steps); query heads
// per workgroup are grouped by 64.
constexpr int kGatherMaxSplit = 1024 + 32;
int gathered_head_groups(int Hq);
DecodePlan decode_plan(int B, int Hq, int Hkv, int Sq, int Sk_max, int dk, int dv);
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);
// Gathered mode's split pass (decode_gathered.hip): bf16 O_s / l_s rows into ws_o, (max, sum) into ws_ml.
hipError_t launch_gathered_split(const DecodeArgs& a, const DecodePlan& plan, uint16_t* ws_o, float* ws_ml,
                                 hipStream_t stream);

// Block dequantization to fp16: fmt 0 = q8_0 (34-byte blocks), 1 = q4_0 (18-byte blocks).
hipError_t launch_dequant(const void* src, int fmt, void* dst, long long n_blocks, hipStream_t stream);

// MLA decode tail: u = bf16(per-head out-absorb of o_lat), y = u @ w_o (split-K, fp32 partials).
struct TailArgs {
    const void* o_lat;     // bf16 [T, H, R]
    const void* w_absorb;  // bf16 [H, DV, R]
    const void* w_o;       // bf16 [H * DV, N]
    void* y;               // [T, N], bf16 or fp32
    int y_f32;
    int T, H, R, DV, N;
    void* workspace;
};

struct TailPlan {
    int ks;           // K slices of the o-projection grid
    int kslice;       // K rows per slice (a multiple of 64)
    bool wn;          // o-projection workgroups span 512 columns (waves on N) instead of splitting K
    size_t u_bytes;   // bf16 u [T, H * DV], rounded up to 256 bytes
    size_t ws_bytes;  // u + fp32 partials [ks, T, N]
};

TailPlan tail_plan(int T, int H, int R, int DV, int N);
hipError_t launch_mla_tail(const TailArgs& a, const TailPlan& plan, hipStream_t stream);

}  // namespace attn
