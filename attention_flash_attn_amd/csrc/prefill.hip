// Fused prefill attention for gfx950: one workgroup per (128-query tile, query head, batch).
//
// Follows the tensor kernel of the "ggml-metal: FA tensor path: gate to the
// (256, 256) shape" page in what it computes (raw QK^T product, scale, softcap,
// mask, online softmax with running max and sum, P kept in registers as the
// operand of the PV product, sinks merged at the end, O / S with a zero-sum row
// written as 0, GQA head map h / (Hq / Hkv)) but not in how: the design here is
// built around CDNA4's 32x32x16 bf16 MFMA and wave64.
//
//  * Each of the 4 waves owns 32 query rows. The score tile is computed
//    transposed, S^T = K Q^T, so every lane holds the scores of ONE query
//    (column lane%32) for 16 keys per 32-key block: the row max is an
//    in-register reduction plus one permlane32 swap, the row sum needs no
//    cross-lane step until the end, and the O rescale factor is lane-local.
//    (The same idea as the key-major score layout on the "MLA Decode Attention
//    Kernel API Reference" page, Notes.)
//  * O is accumulated transposed too, O^T += V^T P^T: the S^T accumulator
//    registers of a lane are exactly its P^T operand for the PV MFMA (after a
//    bf16 pack), so P never leaves registers. The key order inside a 16-key
//    step is permuted to match; the V^T operand is read from LDS with
//    ds_read_b64_tr_b16 in that same key order.
//  * K/V tiles of BN keys are staged in LDS with coalesced 16-byte loads,
//    double-buffered (next tile's global loads are in flight during the
//    current tile's math), XOR-swizzled by 16-byte chunk.
//  * Scores are kept in log2 units (scale * log2 e folded into one multiply)
//    so every exponential is one v_exp_f32.
//  * Causal: tiles past the workgroup's last visible key are never loaded,
//    a wave skips tiles wholly above its diagonal, and only tiles crossing the
//    diagonal or the end of the keys evaluate the mask.
#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {
namespace {

struct PrefillParams {
    const uint16_t* __restrict__ q;
    const uint16_t* __restrict__ k;
    const uint16_t* __restrict__ v;
    void* __restrict__ o;
    float* __restrict__ lse;
    const float* __restrict__ sinks;
    int B, Hq, Hkv, Sq, Sk, group, nqt;
    float c_score;  // scale * log2 e                (softcap off)
    float c_tanh;   // 2 * scale / softcap * log2 e  (softcap on: exponent of e^{2y})
    float c_cap;    // softcap * log2 e
    int causal;
    int softcap_on;
};

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup

template <int DK, int DV, int BN, bool OF32>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
    constexpr int DVP = DV < 32 ? 32 : DV;  // V rows padded to a whole 32-row block of O^T
    constexpr int NCK = DK / 8;             // 16-byte chunks per K row
    constexpr int NCV = DVP / 8;            // 16-byte chunks per (padded) V row in LDS
    constexpr int NCVG = DV / 8;            // 16-byte chunks per V row in memory
    constexpr int KB = BN / 32;             // 32-key blocks per tile
    constexpr int KK = DK / 16;             // k-steps of the QK product
    constexpr int DB = DVP / 32;            // 32-row blocks of O^T
    constexpr int K_BYTES = BN * DK * 2;
    constexpr int V_BYTES = BN * DVP * 2;
    constexpr int STAGE = K_BYTES + V_BYTES;
    constexpr int LK = (BN * NCK + kThreads - 1) / kThreads;
    constexpr int LV = (BN * NCVG + kThreads - 1) / kThreads;
    static_assert(DK % 16 == 0 && DV % 16 == 0 && BN % 32 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int col = lane & 31;

    const int HB = p.Hq * p.B;
    const int bid = blockIdx.x;
    const int qt = p.nqt - 1 - bid / HB;  // heaviest (latest) query tiles first
    const int hb = bid % HB;
    const int h = hb % p.Hq;
    const int b = hb / p.Hq;
    const int g = h / p.group;
    const int q0 = qt * kBM + wave * 32;
    const int qi = q0 + col;
    const int shift = p.Sk - p.Sq;

    if constexpr (DVP != DV) {
        // padding columns of V must read as zero; tile loads never write them
        for (int i = tid; i < 2 * STAGE / 16; i += kThreads) {
            const int s = i / (STAGE / 16), off = (i % (STAGE / 16)) * 16;
            if (off >= K_BYTES) *(u32x4*)(smem + s * STAGE + off) = u32x4{0, 0, 0, 0};
        }
    }

    // this lane's Q fragments: row qi, chunks 2*kk + half
    bf16x8 qf[KK];
    {
        const uint16_t* qrow = p.q + ((size_t)(b * p.Sq + qi) * p.Hq + h) * DK;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            u32x4 w = {0, 0, 0, 0};
            if (qi < p.Sq) w = *(const u32x4*)(qrow + (2 * kk + half) * 8);
            qf[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }

    int kv_end = p.Sk;
    if (p.causal) kv_end = min(p.Sk, qt * kBM + kBM + shift);
    const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;

    const uint16_t* kbase = p.k + (size_t)b * p.Sk * p.Hkv * DK + (size_t)g * DK;
    const uint16_t* vbase = p.v + (size_t)b * p.Sk * p.Hkv * DV + (size_t)g * DV;
    const size_t kstride = (size_t)p.Hkv * DK, vstride = (size_t)p.Hkv * DV;

    u32x4 kreg[LK], vreg[LV];
    auto gload = [&](int t) {
#pragma unroll
        for (int i = 0; i < LK; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx / NCK, c = idx % NCK;
            const int key = t * BN + r;
            u32x4 w = {0, 0, 0, 0};
            if (idx < BN * NCK && key < p.Sk) w = *(const u32x4*)(kbase + key * kstride + c * 8);
            kreg[i] = w;
        }
#pragma unroll
        for (int i = 0; i < LV; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx / NCVG, c = idx % NCVG;
            const int key = t * BN + r;
            u32x4 w = {0, 0, 0, 0};
            if (idx < BN * NCVG && key < p.Sk) w = *(const u32x4*)(vbase + key * vstride + c * 8);
            vreg[i] = w;
        }
    };
    auto lstore = [&](int s) {
        char* kt = smem + s * STAGE;
        char* vt = kt + K_BYTES;
#pragma unroll
        for (int i = 0; i < LK; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx / NCK, c = idx % NCK;
            if (idx < BN * NCK) *(u32x4*)(kt + r * (DK * 2) + ((c ^ swz<NCK>(r)) * 16)) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < LV; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx / NCVG, c = idx % NCVG;
            if (idx < BN * NCVG) *(u32x4*)(vt + r * (DVP * 2) + ((c ^ swz<NCV>(r)) * 16)) = vreg[i];
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) oacc[d] = f32x16{};
    float m_run = -INFINITY;  // running max of this lane's query (log2 units), same in both halves
    float l_run = 0.f;        // this lane's share of the running sum (its half of each key block)

    if (ntiles > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int s = t & 1;
        if (t + 1 < ntiles) gload(t + 1);
        const int key0 = t * BN;
        const bool skip = p.causal && (key0 > q0 + 31 + shift);  // wave-uniform
        if (!skip) {
            const char* kt = smem + s * STAGE;
            const char* vt = kt + K_BYTES;

            // S^T = K Q^T for this tile
            f32x16 sacc[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                sacc[kb] = f32x16{};
                const int r = kb * 32 + col;
                const char* krow = kt + r * (DK * 2);
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const int c = 2 * kk + half;
                    const bf16x8 a = *(const bf16x8*)(krow + ((c ^ swz<NCK>(r)) * 16));
                    sacc[kb] = mfma32x32x16(a, qf[kk], sacc[kb]);
                }
            }

            // score transform (scale, softcap) into log2 units, mask, tile max
            const bool need_mask = (key0 + BN > p.Sk) || (p.causal && key0 + BN - 1 > q0 + shift);
            const int lim = p.causal ? min(p.Sk - 1, qi + shift) : p.Sk - 1;
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float x = sacc[kb][i];
                    if (p.softcap_on) {
                        // cap * tanh(y), y = scale*x/cap; tanh(y) = 1 - 2 / (e^{2y} + 1)
                        const float e = exp2_fast(x * p.c_tanh);
                        x = (1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f)) * p.c_cap;
                    } else {
                        x *= p.c_score;
                    }
                    if (need_mask) {
                        const int key = key0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
                        if (key > lim) x = -INFINITY;
                    }
                    sacc[kb][i] = x;
                    tmax = fmaxf(tmax, x);
                }
            }
            tmax = halfwave_max(tmax);
            const float m_new = fmaxf(m_run, tmax);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2_fast(m_run - m_use);
            m_run = m_new;

            // P = 2^(x - m) rounded to bf16 and packed as the PV operand; the
            // running sum uses the rounded values so O stays a convex combination
            uint32_t pk[KB][8];
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t w = pack_bf16x2(exp2_fast(sacc[kb][2 * j] - m_use),
                                                   exp2_fast(sacc[kb][2 * j + 1] - m_use));
                    pk[kb][j] = w;
                    psum += bf16lo_to_f32(w) + bf16hi_to_f32(w);
                }
            }
            l_run = l_run * alpha + psum;
#pragma unroll
            for (int d = 0; d < DB; ++d) oacc[d] *= alpha;

            // O^T += V^T P^T, 16 keys per MFMA
            const int trow = (lane & 15) >> 2;                       // row within the 4-row block
            const int tcol = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;  // column within the 32-col block
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const u32x4 pw = {pk[kb][4 * jj], pk[kb][4 * jj + 1], pk[kb][4 * jj + 2], pk[kb][4 * jj + 3]};
                    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
                    const int ra = kb * 32 + 16 * jj + half * 4 + trow;
                    const int rb = ra + 8;
#pragma unroll
                    for (int d = 0; d < DB; ++d) {
                        const int dc = d * 32 + tcol;
                        const int ch = dc >> 3, within = (dc & 7) * 2;
                        const bf16x4 va = lds_read_tr16(vt + ra * (DVP * 2) + ((ch ^ swz<NCV>(ra)) * 16) + within);
                        const bf16x4 vb = lds_read_tr16(vt + rb * (DVP * 2) + ((ch ^ swz<NCV>(rb)) * 16) + within);
                        const bf16x8 a = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
                        oacc[d] = mfma32x32x16(a, pb, oacc[d]);
                    }
                }
            }
        }
        if (t + 1 < ntiles) lstore(s ^ 1);
        __syncthreads();
    }

    // epilogue: sinks, normalisation, store
    const float l_tot = halfwave_sum(l_run);
    const bool has_sink = p.sinks != nullptr;
    const float sink2 = has_sink ? p.sinks[h] * kLog2e : -INFINITY;
    const float m2 = fmaxf(m_run, sink2);
    const float m2u = (m2 == -INFINITY) ? 0.f : m2;
    const float fac = exp2_fast(m_run - m2u);
    const float den = l_tot * fac + (has_sink ? exp2_fast(sink2 - m2u) : 0.f);
    const float inv = den > 0.f ? fac / den : 0.f;
    if (qi < p.Sq) {
        if (p.lse != nullptr && half == 0)
            p.lse[((size_t)b * p.Hq + h) * p.Sq + qi] =
                den > 0.f ? (m2u + __builtin_amdgcn_logf(den)) * kLn2 : -INFINITY;
        const size_t obase = ((size_t)(b * p.Sq + qi) * p.Hq + h) * DV;
#pragma unroll
        for (int d = 0; d < DB; ++d) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int dd = d * 32 + a4 * 8 + half * 4;
                if (dd < DV) {
                    const float v0 = oacc[d][4 * a4] * inv, v1 = oacc[d][4 * a4 + 1] * inv;
                    const float v2 = oacc[d][4 * a4 + 2] * inv, v3 = oacc[d][4 * a4 + 3] * inv;
                    if constexpr (OF32) {
                        *(f32x4*)((float*)p.o + obase + dd) = f32x4{v0, v1, v2, v3};
                    } else {
                        *(u32x2*)((uint16_t*)p.o + obase + dd) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                    }
                }
            }
        }
    }
}

template <int DK, int DV, int BN>
hipError_t launch_inst(const PrefillParams& p, bool of32, hipStream_t stream) {
    const dim3 grid((unsigned)(p.nqt * p.Hq * p.B)), block(kThreads);
    if (of32)
        hipLaunchKernelGGL((prefill_kernel<DK, DV, BN, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_kernel<DK, DV, BN, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace

bool prefill_supported(int dk, int dv) {
    switch (dk * 1000 + dv) {
        case 16016: case 32032: case 64064: case 96096: case 128128:
        case 192192: case 256256: case 192128:
            return true;
        default:
            return false;
    }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    PrefillParams p;
    p.q = (const uint16_t*)a.q;
    p.k = (const uint16_t*)a.k;
    p.v = (const uint16_t*)a.v;
    p.o = a.o;
    p.lse = a.lse;
    p.sinks = a.sinks;
    p.B = a.B;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.Sq = a.Sq;
    p.Sk = a.Sk;
    p.group = a.Hq / a.Hkv;
    p.nqt = (a.Sq + kBM - 1) / kBM;
    p.c_score = a.scale * kLog2e;
    p.softcap_on = a.softcap != 0.f;
    p.c_tanh = p.softcap_on ? 2.f * a.scale / a.softcap * kLog2e : 0.f;
    p.c_cap = a.softcap * kLog2e;
    p.causal = a.causal;
    const bool of32 = a.o_f32 != 0;
    switch (a.dk * 1000 + a.dv) {
        case 16016: return launch_inst<16, 16, 64>(p, of32, stream);
        case 32032: return launch_inst<32, 32, 64>(p, of32, stream);
        case 64064: return launch_inst<64, 64, 64>(p, of32, stream);
        case 96096: return launch_inst<96, 96, 64>(p, of32, stream);
        case 128128: return launch_inst<128, 128, 64>(p, of32, stream);
        case 192192: return launch_inst<192, 192, 64>(p, of32, stream);
        case 256256: return launch_inst<256, 256, 64>(p, of32, stream);
        case 192128: return launch_inst<192, 128, 64>(p, of32, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
