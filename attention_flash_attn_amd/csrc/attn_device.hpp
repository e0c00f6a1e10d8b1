// Device helpers shared by the attention kernels (gfx950 / CDNA4, wave64).
//
// MFMA operand maps used throughout (verified on the hardware):
//   v_mfma_f32_32x32x16_bf16  A[32 x 16], B[16 x 32], D[32 x 32]
//     lane l supplies A[row l%32][k (l/32)*8 + e] and B[k (l/32)*8 + e][col l%32], e = 0..7
//     lane l holds   D[row (i/4)*8 + (l/32)*4 + i%4][col l%32] in accumulator i = 0..15
//   ds_read_b64_tr_b16 (per 16-lane group): lane 4r + c points at 4 bf16 of row r,
//     columns 4c..4c+3 of a 4 x 16 block; lane i receives column i, rows 0..3.
//   v_mfma_f32_16x16x32_bf16  A[16 x 32], B[32 x 16], D[16 x 16]
//     lane l supplies A[row l%16][k (l/16)*8 + e] and B[k (l/16)*8 + e][col l%16], e = 0..7
//     lane l holds   D[row (l/16)*4 + i][col l%16] in accumulator i = 0..3
//   v_permlane32_swap(x, x) returns {x[l%32], x[l%32 + 32]} in some order on
//     every lane, so max/sum of the pair combines the two half-waves;
//     v_permlane16_swap(x, x) does the same for lanes l and l^16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define ATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum of a value across the two half-waves (lanes l and l^32).
__device__ __forceinline__ float halfwave_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halfwave_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max / sum across the four 16-lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float quarterwave_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return halfwave_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float quarterwave_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return halfwave_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Round two floats to bf16 (nearest even) and pack them, low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// v_dot2_f32_bf16: acc + lo(w) + hi(w) for a packed bf16 pair (sum of two rounded probabilities).
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

// ---- operand element type: bf16 (F16 = false) or IEEE fp16 (F16 = true) ----
// 16-bit operands travel as bf16x8 bit patterns and are reinterpreted for the
// f16 MFMAs (same shapes and rates on gfx950).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <bool F16>
__device__ __forceinline__ f32x16 mma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <bool F16>
__device__ __forceinline__ f32x4 mma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Round two floats to the operand type (nearest even) and pack them, low half first.
template <bool F16>
__device__ __forceinline__ uint32_t pack_op2(float lo, float hi) {
    if constexpr (F16) {
        f16x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        return pack_bf16x2(lo, hi);
    }
}
// acc + lo(w) + hi(w) for a packed pair of the operand type (v_dot2 with ones).
template <bool F16>
__device__ __forceinline__ float add_op2(uint32_t w, float acc) {
    if constexpr (F16) {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
    } else {
        return add_bf16x2(w, acc);
    }
}

// Element type of a query tensor: 0 = bf16, 1 = fp32, 2 = fp16 (the ABI's codes).
// Loads 8 consecutive elements at p (element index `idx`) as the MFMA operand type.
template <bool F16>
__device__ __forceinline__ bf16x8 load_q8(const void* p, size_t idx, int qtype) {
    if (qtype == 1) {
        const f32x4 a = *(const f32x4*)((const float*)p + idx);
        const f32x4 b = *(const f32x4*)((const float*)p + idx + 4);
        const u32x4 w = {pack_op2<F16>(a[0], a[1]), pack_op2<F16>(a[2], a[3]), pack_op2<F16>(b[0], b[1]),
                         pack_op2<F16>(b[2], b[3])};
        return __builtin_bit_cast(bf16x8, w);
    }
    if (qtype == 2 && !F16) {  // fp16 -> bf16 (read as an fp16 vector and widened element-wise)
        const f16x8 hv = *(const f16x8*)((const _Float16*)p + idx);
        const u32x4 w = {pack_op2<F16>((float)hv[0], (float)hv[1]), pack_op2<F16>((float)hv[2], (float)hv[3]),
                         pack_op2<F16>((float)hv[4], (float)hv[5]), pack_op2<F16>((float)hv[6], (float)hv[7])};
        return __builtin_bit_cast(bf16x8, w);
    }
    const u32x4 raw = *(const u32x4*)((const uint16_t*)p + idx);
    if (qtype == 0 && F16) {  // bf16 -> fp16
        const u32x4 w = {pack_op2<F16>(bf16lo_to_f32(raw[0]), bf16hi_to_f32(raw[0])),
                         pack_op2<F16>(bf16lo_to_f32(raw[1]), bf16hi_to_f32(raw[1])),
                         pack_op2<F16>(bf16lo_to_f32(raw[2]), bf16hi_to_f32(raw[2])),
                         pack_op2<F16>(bf16lo_to_f32(raw[3]), bf16hi_to_f32(raw[3]))};
        return __builtin_bit_cast(bf16x8, w);
    }
    return __builtin_bit_cast(bf16x8, raw);  // already the operand type
}

// Direct HBM -> LDS copy of 16 bytes per lane: lane i writes lds_base + 16 * i
// (lds_base must be wave-uniform). Inactive lanes write nothing.
__device__ __forceinline__ void load_lds16(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (ATTN_LDS void*)(reinterpret_cast<uintptr_t>(lds_base)), 16, 0, 0);
}

// The same copy with the non-temporal hint (cache-policy bit nt): for data read once, such as
// a KV cache streamed by decode, so it does not displace reused lines from the caches.
__device__ __forceinline__ void load_lds16_nt(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (ATTN_LDS void*)(reinterpret_cast<uintptr_t>(lds_base)), 16, 0, 2);
}

// Buffer resource (V#) over [base, base + bytes): offsets >= bytes are out of range.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_buffer(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = (int32_t)(uint32_t)a;
    r[1] = (int32_t)(uint32_t)(a >> 32);  // stride 0
    r[2] = (int32_t)bytes;                // num_records (bytes)
    r[3] = 0x00020000;                    // gfx9-family data format word
    return r;
}
constexpr uint32_t kOobOffset = 0x80000000u;  // an offset that is always out of range

extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(i32x4 rsrc, ATTN_LDS uint32_t* lds, int size, int voffset,
                                                           int soffset, int offset,
                                                           int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
// Buffer -> LDS copy of 16 bytes per lane (lane i writes lds_base + 16 * i); an out-of-range
// offset must not be relied on to write anything.
__device__ __forceinline__ void buffer_load_lds16(i32x4 rsrc, uint32_t voffset, void* lds_base) {
    llvm_amdgcn_raw_buffer_load_lds(rsrc, (ATTN_LDS uint32_t*)(reinterpret_cast<uintptr_t>(lds_base)), 16,
                                    (int)voffset, 0, 0, 0);
}
// Wait until this wave's outstanding vector-memory loads (incl. direct-to-LDS) completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposing LDS read: 4 bf16 (one column of a 4 x 16 block per lane, see above).
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (ATTN_LDS bf16x4*)(reinterpret_cast<uintptr_t>(p)));
}

// The same read through an LDS-typed pointer. With the pointer's provenance kept (no
// integer round trip) the compiler can tell the read from direct-to-LDS copies into other
// LDS objects, instead of waiting for every copy in flight before it.
__device__ __forceinline__ bf16x4 lds_read_tr16_l(const ATTN_LDS char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4*)p);
}

// 16-byte chunk swizzle of LDS rows holding NCH chunks. The LDS serves 256
// bytes per cycle (64 banks of 4 bytes); a row's logical chunk c is stored at
// c ^ swz(r) so that the reads each kernel issues are conflict-free:
//  * 32x32 MFMA operands (MF16 = false): a 128-bit read of one chunk by 16
//    consecutive rows, and a transposing read of 4 aligned rows x 64 bytes;
//  * 16x16 MFMA operands (MF16 = true): a 128-bit read of one chunk by 16
//    consecutive rows, and a transposing read of 8 aligned rows x 32 bytes.
// Rows whose pitch is a multiple of 256 bytes use a 4-bit XOR; pitches that
// are 128 bytes mod 256 (consecutive rows start half a bank row apart) a
// 3-bit XOR; the swizzle never leaves the row.
template <int NCH, bool MF16 = false>
__device__ __forceinline__ int swz(int r) {
    constexpr int pitch = NCH * 16;
    if constexpr (pitch % 256 == 0) {
        return MF16 ? (((r & 7) << 1) | ((r >> 3) & 1)) : (((r & 3) << 2) | ((r >> 2) & 3));
    } else if constexpr (pitch % 128 == 0) {
        return MF16 ? ((((r >> 1) & 3) << 1) | ((r >> 3) & 1)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
    } else {
        constexpr int mask = (NCH % 4 == 0) ? 3 : (NCH % 2 == 0) ? 1 : 0;
        return (((r & 3) << 1) | ((r >> 2) & 1)) & mask;
    }
}

}  // namespace attn
