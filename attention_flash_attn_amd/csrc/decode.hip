// Split-KV decode attention for gfx950: per-split partial results, then a log-sum-exp combine.
//
// Paged mode: the keys of sequence b are read through its block table (logical
// key j -> slot j % bs of physical block table[b][j / bs]), as in the paged
// cache of the "MLA Decode Attention Kernel API Reference" page (parameters:
// kv_cache laid out [n_blocks, 1, block_size, row]). One wavefront per
// (split, KV head, sequence) computes, over its range of keys, the running max
// m, the running sum l and the unnormalised O for every query row that reads
// this KV head (the whole GQA group: the group fills the MFMA's query columns,
// the batching lesson of that page's Notes). The combine pass merges the
// splits with the identity used for sinks in the fa.metal tensor kernel of the
// "ggml-metal: FA tensor path" page (final block): for M = max_s m_s,
//     l = sum_s l_s e^{m_s - M},   O = sum_s O_s e^{m_s - M},
// then adds the sink term and divides.
//
// Scores use the same S^T = K Q^T / O^T += V^T P^T register layout as the
// prefill kernel (one query per lane column); K fragments are loaded straight
// from HBM into MFMA operand registers (16-byte vectors, whole rows consumed by
// one wave), V goes through a small LDS block for the transposing read.
#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {
namespace {

constexpr int kSplitLen = 512;  // keys per split (16 steps of 32 keys)

struct SplitParams {
    const uint16_t* __restrict__ q;
    const uint16_t* __restrict__ kc;
    const uint16_t* __restrict__ vc;
    float* __restrict__ ws_o;   // [rows][n_split][dv]
    float* __restrict__ ws_ml;  // [rows][n_split][2]
    const int32_t* __restrict__ block_table;
    const int32_t* __restrict__ seq_lens;
    int B, Hq, Hkv, Sq, group, nq, bs_log2, max_blocks;
    int n_split;
    float c_score, c_tanh, c_cap;
    int causal, softcap_on;
};

template <int DK, int DV>
__global__ __launch_bounds__(64) void decode_paged_split_kernel(SplitParams p) {
    constexpr int DVP = DV < 32 ? 32 : DV;
    constexpr int NCK = DK / 8;
    constexpr int NCV = DVP / 8;
    constexpr int NCVG = DV / 8;
    constexpr int KK = DK / 16;
    constexpr int DB = DVP / 32;
    constexpr int LV = (32 * NCVG + 63) / 64;
    (void)NCK;
    __shared__ __attribute__((aligned(16))) char vl[32 * DVP * 2];

    const int lane = threadIdx.x, half = lane >> 5, col = lane & 31;
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = p.seq_lens[b];
    const int start = split * kSplitLen;
    if (start >= L) return;  // the combine pass only reads splits that start below L
    const int end = min(L, start + kSplitLen);
    const int bs = 1 << p.bs_log2;

    if constexpr (DVP != DV) {
        for (int i = lane; i < 32 * DVP * 2 / 16; i += 64) *(u32x4*)(vl + i * 16) = u32x4{0, 0, 0, 0};
    }

    // query column -> (query row si, head h of this KV group)
    const bool qvalid = col < p.nq;
    const int si = qvalid ? col / p.group : 0;
    const int h = g * p.group + (qvalid ? col % p.group : 0);
    bf16x8 qf[KK];
    {
        const uint16_t* qrow = p.q + ((size_t)(b * p.Sq + si) * p.Hq + h) * DK;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            u32x4 w = {0, 0, 0, 0};
            if (qvalid) w = *(const u32x4*)(qrow + (2 * kk + half) * 8);
            qf[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }
    // last key this query row may see (bottom-right causal), and the split end
    const int lim = min(end - 1, p.causal ? L - p.Sq + si : L - 1);

    const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
    auto row_ptr_k = [&](int key) -> const uint16_t* {
        const int blk = table[key >> p.bs_log2];
        return p.kc + (((size_t)blk * p.Hkv + g) * bs + (key & (bs - 1))) * DK;
    };
    auto row_ptr_v = [&](int key) -> const uint16_t* {
        const int blk = table[key >> p.bs_log2];
        return p.vc + (((size_t)blk * p.Hkv + g) * bs + (key & (bs - 1))) * DV;
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) oacc[d] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const int trow = (lane & 15) >> 2;
    const int tcol = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;

    for (int k0 = start; k0 < end; k0 += 32) {
        // K fragments of key k0 + col, straight into operand registers
        bf16x8 kf[KK];
        {
            const int key = k0 + col;
            const bool ok = key < end;
            const uint16_t* kr = ok ? row_ptr_k(key) : p.kc;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                u32x4 w = {0, 0, 0, 0};
                if (ok) w = *(const u32x4*)(kr + (2 * kk + half) * 8);
                kf[kk] = __builtin_bit_cast(bf16x8, w);
            }
        }
        // V block of 32 keys into LDS (swizzled rows)
        u32x4 vreg[LV];
#pragma unroll
        for (int i = 0; i < LV; ++i) {
            const int idx = lane + i * 64;
            const int r = idx / NCVG, c = idx % NCVG;
            const int key = k0 + r;
            u32x4 w = {0, 0, 0, 0};
            if (idx < 32 * NCVG && key < end) w = *(const u32x4*)(row_ptr_v(key) + c * 8);
            vreg[i] = w;
        }
        __syncthreads();  // previous step's transposing reads are done
#pragma unroll
        for (int i = 0; i < LV; ++i) {
            const int idx = lane + i * 64;
            const int r = idx / NCVG, c = idx % NCVG;
            if (idx < 32 * NCVG) *(u32x4*)(vl + r * (DVP * 2) + ((c ^ swz<NCV>(r)) * 16)) = vreg[i];
        }

        f32x16 sacc = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) sacc = mfma32x32x16(kf[kk], qf[kk], sacc);

        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x = sacc[i];
            if (p.softcap_on) {
                const float e = exp2_fast(x * p.c_tanh);
                x = (1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f)) * p.c_cap;
            } else {
                x *= p.c_score;
            }
            const int key = k0 + (i >> 2) * 8 + half * 4 + (i & 3);
            if (key > lim) x = -INFINITY;
            sacc[i] = x;
            tmax = fmaxf(tmax, x);
        }
        tmax = halfwave_max(tmax);
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - m_use);
        m_run = m_new;
        uint32_t pk[8];
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t w = pack_bf16x2(exp2_fast(sacc[2 * j] - m_use), exp2_fast(sacc[2 * j + 1] - m_use));
            pk[j] = w;
            psum += bf16lo_to_f32(w) + bf16hi_to_f32(w);
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int d = 0; d < DB; ++d) oacc[d] *= alpha;

        __syncthreads();  // V block visible to every lane
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const u32x4 pw = {pk[4 * jj], pk[4 * jj + 1], pk[4 * jj + 2], pk[4 * jj + 3]};
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
            const int ra = 16 * jj + half * 4 + trow;
            const int rb = ra + 8;
#pragma unroll
            for (int d = 0; d < DB; ++d) {
                const int dc = d * 32 + tcol;
                const int ch = dc >> 3, within = (dc & 7) * 2;
                const bf16x4 va = lds_read_tr16(vl + ra * (DVP * 2) + ((ch ^ swz<NCV>(ra)) * 16) + within);
                const bf16x4 vb = lds_read_tr16(vl + rb * (DVP * 2) + ((ch ^ swz<NCV>(rb)) * 16) + within);
                const bf16x8 a = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[d] = mfma32x32x16(a, pb, oacc[d]);
            }
        }
    }

    const float l_tot = halfwave_sum(l_run);
    if (qvalid) {
        const size_t row = (size_t)(b * p.Sq + si) * p.Hq + h;
        const size_t slot = row * p.n_split + split;
        if (half == 0) {
            p.ws_ml[slot * 2] = m_run;
            p.ws_ml[slot * 2 + 1] = l_tot;
        }
        float* op = p.ws_o + slot * DV;
#pragma unroll
        for (int d = 0; d < DB; ++d) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int dd = d * 32 + a4 * 8 + half * 4;
                if (dd < DV)
                    *(f32x4*)(op + dd) = f32x4{oacc[d][4 * a4], oacc[d][4 * a4 + 1], oacc[d][4 * a4 + 2],
                                               oacc[d][4 * a4 + 3]};
            }
        }
    }
}

struct CombineParams {
    const float* __restrict__ ws_o;
    const float* __restrict__ ws_ml;
    const int32_t* __restrict__ seq_lens;  // paged: bounds the splits to read; NULL: all splits
    const float* __restrict__ sinks;
    void* __restrict__ o;
    int Sq, Hq, n_split, split_len, dv;
};

// One wavefront per output row (b, query, head).
template <bool OF32>
__global__ __launch_bounds__(64) void decode_combine_kernel(CombineParams p) {
    const int lane = threadIdx.x;
    const size_t row = blockIdx.x;
    const int h = (int)(row % p.Hq);
    const int b = (int)(row / ((size_t)p.Sq * p.Hq));
    int nv = p.n_split;
    if (p.seq_lens != nullptr) {
        const int L = p.seq_lens[b];
        nv = min(p.n_split, (L + p.split_len - 1) / p.split_len);
    }
    const float* ml = p.ws_ml + row * p.n_split * 2;
    float M = -INFINITY;
    for (int s = lane; s < nv; s += 64) M = fmaxf(M, ml[2 * s]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const bool has_sink = p.sinks != nullptr;
    const float sink2 = has_sink ? p.sinks[h] * kLog2e : -INFINITY;
    const float M2 = fmaxf(M, sink2);
    const float Mu = (M2 == -INFINITY) ? 0.f : M2;
    float l = 0.f;
    for (int s = lane; s < nv; s += 64) l += ml[2 * s + 1] * exp2_fast(ml[2 * s] - Mu);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
    if (has_sink) l += exp2_fast(sink2 - Mu);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float* ob = p.ws_o + row * p.n_split * p.dv;
    for (int d = lane * 4; d < p.dv; d += 256) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < nv; ++s) {
            const float w = exp2_fast(ml[2 * s] - Mu);
            if (w != 0.f) acc += w * *(const f32x4*)(ob + (size_t)s * p.dv + d);
        }
        acc *= inv;
        if constexpr (OF32) {
            *(f32x4*)((float*)p.o + row * p.dv + d) = acc;
        } else {
            *(u32x2*)((uint16_t*)p.o + row * p.dv + d) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
        }
    }
}

template <int DK, int DV>
hipError_t launch_paged(const SplitParams& sp, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((decode_paged_split_kernel<DK, DV>), grid, dim3(64), 0, stream, sp);
    return hipGetLastError();
}

}  // namespace

bool decode_supported(int dk, int dv, bool gathered) {
    if (gathered) return false;
    switch (dk * 1000 + dv) {
        case 16016: case 32032: case 64064: case 96096: case 128128:
        case 192192: case 256256: case 192128:
            return true;
        default:
            return false;
    }
}

DecodePlan decode_plan(int B, int Hq, int Hkv, int Sq, int Sk_max, int dk, int dv) {
    (void)Hkv;
    (void)dk;
    DecodePlan pl;
    pl.split_len = kSplitLen;
    pl.n_split = Sk_max > 0 ? (Sk_max + kSplitLen - 1) / kSplitLen : 1;
    pl.n_rows = B * Sq * Hq;
    pl.ws_bytes = (size_t)pl.n_rows * pl.n_split * ((size_t)dv + 2) * sizeof(float);
    pl.ws_bytes = (pl.ws_bytes + 255) & ~(size_t)255;
    return pl;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
    float* ws_o = (float*)a.workspace;
    float* ws_ml = ws_o + (size_t)pl.n_rows * pl.n_split * a.dv;
    const float kLog2eH = 1.4426950408889634f;

    SplitParams sp;
    sp.q = (const uint16_t*)a.q;
    sp.kc = (const uint16_t*)a.k_cache;
    sp.vc = (const uint16_t*)a.v_cache;
    sp.ws_o = ws_o;
    sp.ws_ml = ws_ml;
    sp.block_table = a.block_table;
    sp.seq_lens = a.seq_lens;
    sp.B = a.B;
    sp.Hq = a.Hq;
    sp.Hkv = a.Hkv;
    sp.Sq = a.Sq;
    sp.group = a.Hq / a.Hkv;
    sp.nq = a.Sq * sp.group;
    int lg = 0;
    while ((1 << lg) < a.block_size) ++lg;
    sp.bs_log2 = lg;
    sp.max_blocks = a.max_blocks;
    sp.n_split = pl.n_split;
    sp.c_score = a.scale * kLog2eH;
    sp.softcap_on = a.softcap != 0.f;
    sp.c_tanh = sp.softcap_on ? 2.f * a.scale / a.softcap * kLog2eH : 0.f;
    sp.c_cap = a.softcap * kLog2eH;
    sp.causal = a.causal;

    const dim3 grid((unsigned)pl.n_split, (unsigned)a.Hkv, (unsigned)a.B);
    hipError_t e;
    switch (a.dk * 1000 + a.dv) {
        case 16016: e = launch_paged<16, 16>(sp, grid, stream); break;
        case 32032: e = launch_paged<32, 32>(sp, grid, stream); break;
        case 64064: e = launch_paged<64, 64>(sp, grid, stream); break;
        case 96096: e = launch_paged<96, 96>(sp, grid, stream); break;
        case 128128: e = launch_paged<128, 128>(sp, grid, stream); break;
        case 192192: e = launch_paged<192, 192>(sp, grid, stream); break;
        case 256256: e = launch_paged<256, 256>(sp, grid, stream); break;
        case 192128: e = launch_paged<192, 128>(sp, grid, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;

    CombineParams cp;
    cp.ws_o = ws_o;
    cp.ws_ml = ws_ml;
    cp.seq_lens = a.seq_lens;
    cp.sinks = a.sinks;
    cp.o = a.o;
    cp.Sq = a.Sq;
    cp.Hq = a.Hq;
    cp.n_split = pl.n_split;
    cp.split_len = pl.split_len;
    cp.dv = a.dv;
    if (a.o_f32)
        hipLaunchKernelGGL((decode_combine_kernel<true>), dim3((unsigned)pl.n_rows), dim3(64), 0, stream, cp);
    else
        hipLaunchKernelGGL((decode_combine_kernel<false>), dim3((unsigned)pl.n_rows), dim3(64), 0, stream, cp);
    return hipGetLastError();
}

}  // namespace attn
