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
// One 256-thread workgroup per 256 blocks: the packed bytes (8704 or 4608,
// 16-byte aligned whenever the buffer is) are staged into LDS with 16-byte
// loads, then thread i expands block i into 64 contiguous output bytes.
#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {
namespace {

constexpr int kBlocksPerWG = 256;

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
    if (tid >= nb) return;

    const uint8_t* b = stage + tid * BYTES;
    const float d = (float)__builtin_bit_cast(_Float16, *(const uint16_t*)b);
    float v[32];
    if constexpr (BYTES == 34) {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = d * (float)(int8_t)b[2 + i];
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int x = b[2 + j];
            v[j] = d * (float)((x & 15) - 8);
            v[j + 16] = d * (float)((x >> 4) - 8);
        }
    }
    uint16_t* o = dst + (blk0 + tid) * 32;
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
        const u32x4 w = {pack_op2<true>(v[i], v[i + 1]), pack_op2<true>(v[i + 2], v[i + 3]),
                         pack_op2<true>(v[i + 4], v[i + 5]), pack_op2<true>(v[i + 6], v[i + 7])};
        *(u32x4*)(o + i) = w;
    }
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
