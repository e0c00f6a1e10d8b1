// MLA decode tail for gfx950: the out-absorb and the o-projection that follow
// MLA decode attention ("MLA Decode Attention Kernel API Reference" page:
// Background, the out_absorb_w and o_proj_w parameters, and Notes, where both
// tails are per-token products against shared weights, batched across tokens).
//
//   u[t, h*DV + v] = bf16( sum_c w_abs[h, v, c] * o_lat[t, h, c] )
//   y[t, n]        = sum_k u[t, k] * w_o[k, n]                  (k = h*DV + v)
//
// At decode sizes both products stream their weights (16 tokens make about 16
// flops per weight byte), so the kernels are built to read every weight byte
// once with many loads in flight, as non-temporal loads (8% faster). They use
// v_mfma_f32_16x16x32_bf16 with the tokens as the 16-row side, fp32
// accumulation, and u rounded to bf16 (nearest even) as the o-projection's
// operand.
//  * absorb: one wave per (head, 16 values of v). Rows of w_abs are contiguous
//    in the latent index, which is the product's contraction index, so both
//    operands load straight from memory as 16-byte fragments.
//  * o-projection: w_o is [K, N] with N contiguous, while an MFMA lane needs a
//    run of 8 consecutive K for one column. Each lane loads 8 rows x 8 columns
//    (eight 16-byte loads; a 16-lane group reads 256 contiguous bytes of a row)
//    and transposes them in registers into the K-runs of its 8 columns, so the
//    weights make no LDS round trip. A workgroup's 4 waves take 4 adjacent
//    128-column strips of the same rows (when N allows; else they split its K
//    range and add their tiles in LDS); the grid splits K into KS slices whose
//    fp32 partial tiles a last pass adds in a fixed order and rounds.
#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {
namespace {

constexpr int kTailCols = 128;  // output columns per o-projection wave

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0}); }

// u rows t0 .. t0 + nt - 1 (nt <= 16 RB). Grid: H * DV / 16 waves.
template <int RB, int NKU>  // NKU: 128-wide latent blocks per loop step (all its loads issued at once)
__global__ __launch_bounds__(64) void absorb_kernel(const uint16_t* __restrict__ o_lat, const uint16_t* __restrict__ wa,
                                                    uint16_t* __restrict__ u, int T, int H, int R, int DV, int t0) {
    const int lane = threadIdx.x, r16 = lane & 15, kg = lane >> 4;
    const int nvb = DV / 16;
    // workgroup -> (head, block of 16 values). With H a multiple of 8, XCD x (= blockIdx % 8)
    // takes heads x, x + 8, ...: the nvb workgroups of a head share one L2, which then serves
    // the head's latent rows to all of them (a head-major order would fetch them on every XCD).
    int h, vb;
    if ((H & 7) == 0) {
        const int j = blockIdx.x >> 3;
        h = (blockIdx.x & 7) + 8 * (j / nvb);
        vb = j % nvb;
    } else {
        h = blockIdx.x / nvb;
        vb = blockIdx.x % nvb;
    }
    const int nt = min(T - t0, RB * 16);
    // B operand: w_abs[h][v = vb*16 + r16][c], 8 consecutive c per lane
    const uint16_t* wrow = wa + ((size_t)h * DV + vb * 16 + r16) * R + kg * 8;
    // A operand: o_lat[t][h][c]; rows past the last token read token t0 and are zeroed
    const uint16_t* arow[RB];
    bool aok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int tl = rb * 16 + r16;
        aok[rb] = tl < nt;
        arow[rb] = o_lat + ((size_t)(t0 + (aok[rb] ? tl : 0)) * H + h) * R + kg * 8;
    }
    f32x4 acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < R; k0 += 128 * NKU) {
        constexpr int NJ = 4 * NKU;
        bf16x8 b[NJ], a[RB][NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) b[j] = __builtin_nontemporal_load((const bf16x8*)(wrow + k0 + j * 32));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < NJ; ++j) a[rb][j] = *(const bf16x8*)(arow[rb] + k0 + j * 32);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) acc[rb] = mma16<false>(aok[rb] ? a[rb][j] : zero8(), b[j], acc[rb]);
    }
    // lane holds tokens rb*16 + kg*4 + i of column v = vb*16 + r16
    const size_t K = (size_t)H * DV;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tl = rb * 16 + kg * 4 + i;
            if (tl < nt) {
                u[(size_t)(t0 + tl) * K + (size_t)h * DV + vb * 16 + r16] =
                    (uint16_t)(pack_bf16x2(acc[rb][i], 0.f) & 0xffffu);
            }
        }
}

// Partial y tiles: part[ks][t][n] for tokens t0 .. t0 + nt - 1, columns
// blockIdx.x * 128 .. + 127, K rows ks * kslice .. + kslice - 1 (blockIdx.y = ks).
constexpr int kTailWaves = 4;  // waves per o-projection workgroup
// WN: the 4 waves take 4 adjacent 128-column strips of the same K rows (a workgroup reads
// 1 KB of every row: measured 20% faster than splitting K, 5.7 TB/s at hidden 7168);
// else (N not a multiple of 512) they split the K rows of one 128-column strip.
template <int RB, bool WN>
__global__ __launch_bounds__(64 * kTailWaves) void oproj_kernel(const uint16_t* __restrict__ u, const uint16_t* __restrict__ wo,
                                                    float* __restrict__ part, int T, int K, int N, int kslice,
                                                    int t0) {
    static_assert(kTailWaves == 4, "the K-split reduction below adds 4 tiles with 256 threads");
    __shared__ float red[WN ? 1 : kTailWaves][16][kTailCols + 4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    const int n0 = WN ? (blockIdx.x * kTailWaves + wave) * kTailCols : blockIdx.x * kTailCols;
    const int ks = blockIdx.y;
    const int kw = WN ? kslice : kslice / kTailWaves;  // K rows of this wave (a multiple of 32)
    const int kbeg = ks * kslice + (WN ? 0 : wave * kw);
    const int nt = min(T - t0, RB * 16);

    // lane: rows kbeg + 32c + 8g + e (e = 0..7) of columns n0 + 8*c16 .. + 7
    const uint16_t* wp = wo + (size_t)(kbeg + 8 * g) * N + n0 + 8 * c16;
    const uint16_t* ap[RB];
    bool aok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int tl = rb * 16 + c16;
        aok[rb] = tl < nt;
        ap[rb] = u + (size_t)(t0 + (aok[rb] ? tl : 0)) * K + kbeg + 8 * g;
    }
    f32x4 acc[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 w0[8], w1[8], w2[8];
    bf16x8 a0[RB], a1[RB], a2[RB];
    auto load = [&](int c, u32x4 (&w)[8], bf16x8 (&a)[RB]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = __builtin_nontemporal_load((const u32x4*)(wp + (size_t)(c * 32 + e) * N));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) a[rb] = *(const bf16x8*)(ap[rb] + c * 32);
    };
    // column j of the lane's 8 x 8 block as the K-run operand (rows 0..7 = the lane's K index 8g + e)
    auto compute = [&](const u32x4 (&w)[8], const bf16x8 (&a)[RB]) {
        bf16x8 av[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) av[rb] = aok[rb] ? a[rb] : zero8();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int p = j >> 1;
            u32x4 bw;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                bw[m] = (j & 1) ? ((w[2 * m][p] >> 16) | (w[2 * m + 1][p] & 0xffff0000u))
                                : ((w[2 * m][p] & 0xffffu) | (w[2 * m + 1][p] << 16));
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc[rb][j] = mma16<false>(av[rb], __builtin_bit_cast(bf16x8, bw), acc[rb][j]);
        }
    };
    // three chunks in a register ring: two are in flight while one is multiplied
    const int nch = kw / 32;
    load(0, w0, a0);
    if (1 < nch) load(1, w1, a1);
    for (int c = 0; c < nch; c += 3) {
        if (c + 2 < nch) load(c + 2, w2, a2);
        compute(w0, a0);
        if (c + 3 < nch) load(c + 3, w0, a0);
        if (c + 1 < nch) compute(w1, a1);
        if (c + 4 < nch) load(c + 4, w1, a1);
        if (c + 2 < nch) compute(w2, a2);
    }

    if constexpr (WN) {  // lane holds tokens rb*16 + g*4 + i of columns n0 + 8*c16 + j
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tl = rb * 16 + g * 4 + i;
                if (tl < nt) {
                    float* dst = part + ((size_t)ks * T + t0 + tl) * N + n0 + 8 * c16;
                    *(f32x4*)dst = f32x4{acc[rb][0][i], acc[rb][1][i], acc[rb][2][i], acc[rb][3][i]};
                    *(f32x4*)(dst + 4) = f32x4{acc[rb][4][i], acc[rb][5][i], acc[rb][6][i], acc[rb][7][i]};
                }
            }
        return;
    }
    // add the 4 waves' tiles, one 16-token block at a time; lane holds tokens
    // g*4 + i of column 8*c16 + j
    const int tl_r = tid >> 4, cc = (tid & 15) * 8;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][g * 4 + i][8 * c16 + j] = acc[rb][j][i];
        __syncthreads();
        const int tl = rb * 16 + tl_r;
        if (tl < nt) {
            f32x4 s0, s1;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s0[q] = ((red[0][tl_r][cc + q] + red[1][tl_r][cc + q]) + red[2][tl_r][cc + q]) + red[3][tl_r][cc + q];
                s1[q] = ((red[0][tl_r][cc + 4 + q] + red[1][tl_r][cc + 4 + q]) + red[2][tl_r][cc + 4 + q]) +
                        red[3][tl_r][cc + 4 + q];
            }
            float* dst = part + ((size_t)ks * T + t0 + tl) * N + n0 + cc;
            *(f32x4*)dst = s0;
            *(f32x4*)(dst + 4) = s1;
        }
        __syncthreads();
    }
}

// y = sum over the KS slices (in slice order), rounded to bf16 or kept fp32; 4 columns per thread.
__global__ __launch_bounds__(64) void tail_reduce_kernel(const float* __restrict__ part, void* __restrict__ y,
                                                         int y_f32, long long total4, int KS) {
    const long long i = (long long)blockIdx.x * 64 + threadIdx.x;
    if (i >= total4) return;
    const f32x4* p = (const f32x4*)part;
    f32x4 s = p[i];
    int k = 1;
    for (; k + 8 <= KS; k += 8) {  // 8 loads in flight, added in slice order
        f32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = p[(size_t)(k + j) * total4 + i];
#pragma unroll
        for (int j = 0; j < 8; ++j) s += v[j];
    }
    for (; k < KS; ++k) s += p[(size_t)k * total4 + i];
    if (y_f32)
        ((f32x4*)y)[i] = s;
    else
        ((u32x2*)y)[i] = u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
}

template <int RB>
hipError_t launch_chunk(const TailArgs& a, const TailPlan& pl, uint16_t* u, float* part, int t0, hipStream_t stream) {
    const int K = a.H * a.DV;
    if (a.R % 512 == 0 && RB <= 2)
        hipLaunchKernelGGL((absorb_kernel<RB, 4>), dim3((unsigned)(a.H * (a.DV / 16))), dim3(64), 0, stream,
                           (const uint16_t*)a.o_lat, (const uint16_t*)a.w_absorb, u, a.T, a.H, a.R, a.DV, t0);
    else
        hipLaunchKernelGGL((absorb_kernel<RB, 1>), dim3((unsigned)(a.H * (a.DV / 16))), dim3(64), 0, stream,
                           (const uint16_t*)a.o_lat, (const uint16_t*)a.w_absorb, u, a.T, a.H, a.R, a.DV, t0);
    if (pl.wn)
        hipLaunchKernelGGL((oproj_kernel<RB, true>), dim3((unsigned)(a.N / (kTailWaves * kTailCols)), (unsigned)pl.ks), dim3(64 * kTailWaves),
                           0, stream, (const uint16_t*)u, (const uint16_t*)a.w_o, part, a.T, K, a.N, pl.kslice, t0);
    else
        hipLaunchKernelGGL((oproj_kernel<RB, false>), dim3((unsigned)(a.N / kTailCols), (unsigned)pl.ks), dim3(64 * kTailWaves), 0,
                           stream, (const uint16_t*)u, (const uint16_t*)a.w_o, part, a.T, K, a.N, pl.kslice, t0);
    return hipGetLastError();
}

}  // namespace

TailPlan tail_plan(int T, int H, int R, int DV, int N) {
    (void)R;
    TailPlan pl;
    const long long K = (long long)H * DV;
    pl.wn = N % (kTailWaves * kTailCols) == 0;
    const long long n_tiles = pl.wn ? N / (kTailWaves * kTailCols) : N / kTailCols;
    const long long kmult = pl.wn ? 64 : 256;  // K rows of a slice: every wave keeps >= 2 chunks of 32
    // split K until the grid holds about one workgroup per CU (256): fewer, longer-running
    // workgroups stream faster here than 2-4 per CU, and keep the partial sums small
    int ks = 1;
    while (ks < 256 && K % (kmult * ks * 2) == 0 && n_tiles * ks * 2 <= 256) ks *= 2;
    pl.ks = ks;
    pl.kslice = (int)(K / ks);
    pl.u_bytes = ((size_t)T * K * 2 + 255) / 256 * 256;
    pl.ws_bytes = pl.u_bytes + (size_t)ks * T * N * 4;
    return pl;
}

hipError_t launch_mla_tail(const TailArgs& a, const TailPlan& pl, hipStream_t stream) {
    uint16_t* u = (uint16_t*)a.workspace;
    float* part = (float*)((char*)a.workspace + pl.u_bytes);
    for (int t0 = 0; t0 < a.T; t0 += 64) {
        const int nt = a.T - t0 < 64 ? a.T - t0 : 64;
        hipError_t e;
        if (nt <= 16)
            e = launch_chunk<1>(a, pl, u, part, t0, stream);
        else if (nt <= 32)
            e = launch_chunk<2>(a, pl, u, part, t0, stream);
        else
            e = launch_chunk<4>(a, pl, u, part, t0, stream);
        if (e != hipSuccess) return e;
    }
    const long long total4 = (long long)a.T * a.N / 4;
    hipLaunchKernelGGL(tail_reduce_kernel, dim3((unsigned)((total4 + 63) / 64)), dim3(64), 0, stream,
                       (const float*)part, a.y, a.y_f32, total4, pl.ks);
    return hipGetLastError();
}

}  // namespace attn
