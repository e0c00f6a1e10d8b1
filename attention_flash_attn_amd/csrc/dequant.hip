// Block-dequantization of a quantized KV cache to IEEE fp16: the pre-pass that
// the "ggml-metal: FA tensor path" page runs before its fp16 attention kernels
// when K/V are quantized. Block formats (32 values each, fp16 scale d first,
// blocks packed back to back):
//   q8_0: 34 bytes: d, 32 x int8 q                   value = d * q
//   q4_0: 18 bytes: d, 16 bytes of nibbles           value = d * (q - 8);
//         byte j holds value j (low nibble) and value j + 16 (high nibble)
// d * q is exact in fp32 (11 + 8 significand bits) and is rounded once to fp16
// (nearest even).
//
// One 256-thread workgroup per 64 blocks: the packed bytes (2176 or 1152, 16-byte aligned
// whenever the buffer is) are staged into LDS with 16-byte loads; then thread i expands values
// 8 (i % 4) .. 8 (i % 4) + 7 of block i / 4 into 16 output bytes, so a wave stores 1 KB of
// contiguous output per instruction.
#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {
namespace {

constexpr int kBlocksPerWG = 64;

template <int BYTES>  // 34 (q8_0) or 18 (q4_0)
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                      long long n_blocks) {
    constexpr int WG_BYTES = kBlocksPerWG * BYTES;  // multiple of 16
    static_assert(WG_BYTES % 16 == 0, "workgroup span");
    __shared__ __attribute__((aligned(16))) uint8_t stage[WG_BYTES];

    const int tid = threadIdx.x;
    const long long blk0 = (long long)blockIdx.x * kBlocksPerWG;
    const long long nb = n_blocks - blk0 < kBlocksPerWG ? n_blocks - blk0 : kBlocksPerWG;
    const long long total = nb * BYTES;  // bytes of this workgroup
    const uint8_t* s = src + blk0 * BYTES;
    for (int c = tid; c * 16 < total; c += 256) {
        if (c * 16 + 16 <= total) {
            *(u32x4*)(stage + c * 16) = *(const u32x4*)(s + c * 16);
        } else {
            for (int j = c * 16; j < total; j += 2)  // ragged end: whole 2-byte units
                *(uint16_t*)(stage + j) = *(const uint16_t*)(s + j);
        }
    }
    __syncthreads();
    const int blk = tid >> 2, part = tid & 3;
    if (blk >= nb) return;

    const uint8_t* b = stage + blk * BYTES;  // 2-byte aligned
    const float d = (float)__builtin_bit_cast(_Float16, *(const uint16_t*)b);
    float v[8];
    if constexpr (BYTES == 34) {  // values 8 part .. 8 part + 7: bytes 2 + 8 part ..
        const uint16_t* q = (const uint16_t*)(b + 2 + 8 * part);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w = q[j];
            v[2 * j] = d * (float)(int8_t)(w & 0xff);
            v[2 * j + 1] = d * (float)(int8_t)(w >> 8);
        }
    } else {  // values 0-15: low nibbles of bytes 0-15; values 16-31: high nibbles
        const uint16_t* q = (const uint16_t*)(b + 2 + 8 * (part & 1));
        const int sh = (part >> 1) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w = q[j];
            v[2 * j] = d * (float)((int)((w >> sh) & 15) - 8);
            v[2 * j + 1] = d * (float)((int)((w >> (8 + sh)) & 15) - 8);
        }
    }
    const u32x4 w = {pack_op2<true>(v[0], v[1]), pack_op2<true>(v[2], v[3]), pack_op2<true>(v[4], v[5]),
                     pack_op2<true>(v[6], v[7])};
    *(u32x4*)(dst + (blk0 + blk) * 32 + 8 * part) = w;
}

}  // namespace

hipError_t launch_dequant(const void* src, int fmt, void* dst, long long n_blocks, hipStream_t stream) {
    if (n_blocks <= 0) return hipSuccess;
    const dim3 grid((unsigned)((n_blocks + kBlocksPerWG - 1) / kBlocksPerWG));
    if (fmt == 0)
        hipLaunchKernelGGL((dequant_kernel<34>), grid, dim3(256), 0, stream, (const uint8_t*)src, (uint16_t*)dst,
                           n_blocks);
    else
        hipLaunchKernelGGL((dequant_kernel<18>), grid, dim3(256), 0, stream, (const uint8_t*)src, (uint16_t*)dst,
                           n_blocks);
    return hipGetLastError();
}

}  // namespace attn
