// Fused prefill attention for gfx950: one workgroup per (query tile, query head, batch).
//
// Follows the tensor kernel of the "ggml-metal: FA tensor path: gate to the
// (256, 256) shape" page in what it computes (raw QK^T product, scale, softcap,
// mask, online softmax with running max and sum, P kept in registers as the
// operand of the PV product, sinks merged at the end, O / S with a zero-sum row
// written as 0, GQA head map h / (Hq / Hkv)) but not in how: the design here is
// built around CDNA4's 32x32x16 bf16 MFMA and wave64.
//
//  * Each wave owns 32 query rows. The score tile is computed transposed,
//    S^T = K Q^T, so every lane holds the scores of ONE query (column
//    lane%32) for 16 keys per 32-key block: the row max is an in-register
//    reduction plus one permlane32 swap, the row sum needs no cross-lane step
//    until the end, and the O rescale factor is lane-local. (The key-major
//    score layout of the "MLA Decode Attention Kernel API Reference" page,
//    Notes, is the same idea.)
//  * O is accumulated transposed too, O^T += V^T P^T: the S^T accumulator
//    registers of a lane are exactly its P^T operand for the PV MFMA (after a
//    bf16 pack), so P never leaves registers. The key order inside a 16-key
//    step is permuted to match; the V^T operand is read from LDS with
//    ds_read_b64_tr_b16 in that same key order.
//  * K/V tiles of BN keys go HBM -> LDS directly (buffer_load ... lds, 16
//    bytes per lane, 1 KB per wave instruction), double-buffered: tile t+1 is
//    in flight while tile t is computed; one barrier per tile. The LDS
//    layouts make every fragment read a fixed per-lane base plus an immediate
//    offset, with no bank conflicts.
//  * Scores stay in log2 units (scale * log2 e folded into one FMA with the
//    max) so every exponential is one v_exp_f32. The running max moves only
//    when a tile's max exceeds it by more than 2^8 (O and the sum use the same
//    reference, so the result is unchanged; probabilities stay <= 256), which
//    lets the O rescale be skipped for the whole wave on most tiles.
//  * Row sums add the bf16-rounded probabilities two at a time (v_dot2), so O
//    is an exact convex combination of V rows up to fp32 accumulation.
//  * Additive mask (optional, IEEE fp16 [MB, MH, Sq, stride], head h of batch b
//    reading mask[b % MB][h % MH] as in the page's kernel), times the head's
//    ALiBi slope, is added after the softcap; each wave copies its 32 rows of a
//    tile's mask into LDS with the tile's K/V copies (whole row segments per
//    copy), and each lane reads its row's entries from there.
//  * Causal: tiles past the workgroup's last visible key are never loaded, a
//    wave skips tiles wholly above its diagonal, and only tiles crossing the
//    diagonal or the end of the keys evaluate the mask. Workgroups are
//    ordered heaviest query tile first, with heads spread over the 8 XCDs.
#include <type_traits>

#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {
namespace {

struct PrefillParams {
    const void* __restrict__ q;  // bf16, fp32 or fp16 (q_type), converted to the operand type at load
    const uint16_t* __restrict__ k;
    const uint16_t* __restrict__ v;
    void* __restrict__ o;
    float* __restrict__ lse;
    const float* __restrict__ sinks;
    int B, Hq, Hkv, Sq, Sk, group, nqt;
    float c_score;  // scale * log2 e                (softcap off)
    float c_tanh;   // 2 * scale / softcap * log2 e  (softcap on: exponent of e^{2y})
    float c_cap;    // softcap * log2 e
    int xcd_remap;  // 1: B * Hq is a multiple of 8; 2: also B * Hkv (grouped query heads)
    // additive mask (fp16 bits) and ALiBi
    const uint16_t* __restrict__ mask;
    long long mask_stride;  // elements between query rows
    int mask_batch, mask_heads;
    float max_bias;
    int n_head_log2;
    int q_type;  // 0 bf16, 1 fp32, 2 fp16
};

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Buffer -> LDS copy of 16 bytes per lane as inline assembly, which the compiler does not
// track. Tracked copies of the next tile made the compiler wait for every copy in flight
// before the first transposing V^T read of the current tile (it cannot tell the two stages
// apart), so a tile's copies had only its QK product and softmax to land in. The kernel waits
// for its copies itself (vmcnt(0), then the workgroup barrier) before any read of their
// stage. No output registers; M0 carries the LDS address.
__device__ __forceinline__ void buffer_load_lds16_u(i32x4 rsrc, uint32_t voffset, void* lds_base) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds_base));
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 : : "v"(voffset), "s"(rsrc), "s"(m) : "m0");
}

constexpr float kTau = 8.f;  // lazy-rescale threshold (log2 units)

// LDS fragment reads issued ahead of their MFMA (K: 128-bit reads, V: transposing pairs)
#ifndef ATTN_PF_K
#define ATTN_PF_K 4
#endif
#ifndef ATTN_PF_V
#define ATTN_PF_V 4
#endif

// Tile configurations (keys per tile, waves per workgroup, target waves per SIMD)
#ifndef ATTN_D128_CFG
#define ATTN_D128_CFG 64, 8, 2
#endif
#ifndef ATTN_D256_CFG
#define ATTN_D256_CFG 32, 8, 2
#endif

// F16: K, V (and the MFMA operands, P included) are IEEE fp16 instead of bf16.
template <int DK, int DV, int BN, int NW, int OCC, bool CAUSAL, bool SOFTCAP, bool ADDM, bool F16, bool OF32>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC)))
void prefill_kernel(PrefillParams p) {
    constexpr bool LOG2 = SOFTCAP;  // scores converted to log2 units before the max
    constexpr int NT = NW * 64;
    constexpr int BM = NW * 32;             // query rows per workgroup
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
    constexpr int KSEG = K_BYTES / 1024, VSEG = V_BYTES / 1024;  // 1 KB load segments per tile
    static_assert(DK % 16 == 0 && DV % 16 == 0 && BN % 32 == 0, "tile shape");
    static_assert(K_BYTES % 1024 == 0 && V_BYTES % 1024 == 0, "tile must split into 1 KB segments");

    // Copies of the next tile untracked by the compiler (head dims <= 128, and d = 256 without
    // masks; see buffer_load_lds16_u). At d <= 128, with the tile's whole period to land in,
    // the causal prefill at B=2, H=32, 4096^2, d=128 ran 282-286 us against 299-311 us after a
    // 2 GiB cache flush, and 264 against 266-270 us warm. At d = 256 untracked copies issued at
    // the top of the tile were 1.8% slower (GQA 64:8, 4096^2: 928 against 912 us, warm): their
    // LDS writes then meet the fragment reads. Without the causal mask, d = 256 issues them
    // untracked after the QK product instead (LATE), so they land during the softmax: 931-936
    // against 940-947 us; the causal instances keep the tracked form (with LATE 555-559 against
    // 548-550 us), and so do the masked ones (not measured with LATE).
    constexpr bool LATE = DK == 256 && !CAUSAL && !ADDM;
    constexpr bool UNTRACKED = DK <= 128 || LATE;
    auto copy16 = [](i32x4 rsrc, uint32_t voffset, void* lds) {
        if constexpr (UNTRACKED)
            buffer_load_lds16_u(rsrc, voffset, lds);
        else
            buffer_load_lds16(rsrc, voffset, lds);
    };

    // additive mask (ADDM): each wave's 32 query rows x BN keys of fp16 per stage
    constexpr int MT = 32 * BN * 2;
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE + (ADDM ? 2 * NW * MT : 0)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int col = lane & 31;

    // workgroup -> (query tile, head, batch): heaviest tiles first; with
    // xcd_remap 1, XCD x (= blockIdx % 8) works on heads x, x+8, ...; with 2, on
    // the KV groups x, x+8, ... (every query head of a group on one XCD, whose L2
    // then serves the group's K/V to all of them)
    const int HB = p.Hq * p.B;
    int qt, hb;
    if (p.xcd_remap == 2) {
        const int x = blockIdx.x & 7, j = blockIdx.x >> 3, per = HB >> 3;
        qt = p.nqt - 1 - j / per;
        const int r = j % per, G = p.group;
        const int kg = x + 8 * (r / G);
        hb = (kg / p.Hkv) * p.Hq + (kg % p.Hkv) * G + r % G;
    } else if (p.xcd_remap) {
        const int x = blockIdx.x & 7, j = blockIdx.x >> 3, per = HB >> 3;
        qt = p.nqt - 1 - j / per;
        hb = x + 8 * (j % per);
    } else {
        qt = p.nqt - 1 - blockIdx.x / HB;
        hb = blockIdx.x % HB;
    }
    const int h = hb % p.Hq;
    const int b = hb / p.Hq;
    const int g = h / p.group;
    const int q0 = qt * BM + wave * 32;
    const int qi = q0 + col;
    const int shift = p.Sk - p.Sq;

    int kv_end = p.Sk;
    if (CAUSAL) kv_end = min(p.Sk, qt * BM + BM + shift);
    const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;

    // Rows at or past Sk (and the V padding columns) fall outside the buffer
    // ranges below and are not loaded: start both stages at zero so those LDS
    // rows always hold finite values (zero, or an earlier tile's data); their
    // scores are masked and their probabilities are exactly 0.
    if ((DVP != DV) || (p.Sk % BN) != 0) {
        for (int i = tid; i < 2 * STAGE / 16; i += NT) *(u32x4*)(smem + i * 16) = u32x4{0, 0, 0, 0};
        __syncthreads();
    }

    // K and V of this (batch, KV head) as buffers
    const size_t kstride = (size_t)p.Hkv * DK, vstride = (size_t)p.Hkv * DV;
    const i32x4 krsrc = make_buffer(p.k + (size_t)b * p.Sk * kstride + (size_t)g * DK,
                                    (uint32_t)(((size_t)(p.Sk - 1) * kstride + DK) * 2));
    const i32x4 vrsrc = make_buffer(p.v + (size_t)b * p.Sk * vstride + (size_t)g * DV,
                                    (uint32_t)(((size_t)(p.Sk - 1) * vstride + DV) * 2));

    // issue the direct-to-LDS loads of tile t into stage st (each wave: every NW-th 1 KB segment).
    // LDS layouts (chosen so every fragment read below is the lane's base plus an
    // immediate offset, and both read patterns are bank-conflict free):
    //   K: [DK/16 slices][BN rows][32 B]; the two 16-byte halves of a row swap
    //      when bit 3 of the row is set
    //   V: [DVP/32 blocks][BN rows][64 B]
    constexpr int SEGK = BN * 32 / 1024;  // 1 KB segments per K slice
    constexpr int SEGV = BN * 64 / 1024;  // 1 KB segments per V block
    auto issue = [&](int t, int st) {
        char* sb = smem + st * STAGE;
        const uint32_t kbase_off = (uint32_t)(t * BN) * (uint32_t)(kstride * 2);
        const uint32_t vbase_off = (uint32_t)(t * BN) * (uint32_t)(vstride * 2);
#pragma unroll
        for (int i = 0; i < (KSEG + NW - 1) / NW; ++i) {
            const int s = wave + i * NW;
            if (s < KSEG) {
                const int kk = s / SEGK;
                const int r = (s % SEGK) * 32 + (lane >> 1);
                const int piece = (lane & 1) ^ ((r >> 3) & 1);
                copy16(krsrc, kbase_off + (uint32_t)(r * kstride * 2 + kk * 32 + piece * 16), sb + s * 1024);
            }
        }
#pragma unroll
        for (int i = 0; i < (VSEG + NW - 1) / NW; ++i) {
            const int s = wave + i * NW;
            if (s < VSEG) {
                const int db = s / SEGV;
                const int r = (s % SEGV) * 16 + (lane >> 2);
                const int q = lane & 3;
                const uint32_t vo = (db * 32 + q * 8 < DV)
                                        ? vbase_off + (uint32_t)(r * vstride * 2 + db * 64 + q * 16)
                                        : kOobOffset;
                copy16(vrsrc, vo, sb + K_BYTES + s * 1024);
            }
        }
    };

    if (ntiles > 0) issue(0, 0);

    // this lane's Q fragments: row qi, chunks 2*kk + half
    bf16x8 qf[KK];
    {
        const size_t qrow = (((size_t)b * p.Sq + qi) * p.Hq + h) * DK;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            qf[kk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
            if (qi < p.Sq) qf[kk] = load_q8<F16>(p.q, qrow + (2 * kk + half) * 8, p.q_type);
        }
    }

    // The query fragments must have landed before the tile loops: otherwise the compiler, unable
    // to tell across the back edge whether their loads completed, waits for every load in flight
    // (the next tile's untracked copies included) at their first use in every tile.
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(qf[kk]));

    f32x16 oacc[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) oacc[d] = f32x16{};
    float m_run = -INFINITY;  // reference max of this lane's query (log2 units), same in both halves
    float l_run = 0.f;        // this lane's share of the running sum (its half of each key block)
    const int lim = CAUSAL ? min(p.Sk - 1, qi + shift) : p.Sk - 1;  // last visible key of this row

    // additive mask: the wave's 32 query rows of slab mask[b % MB][h % MH] (rows past Sq read
    // row Sq-1), copied per tile into the wave's own LDS region with the K/V copies of the
    // tile (16-byte chunks, 8 rows per 1 KB copy, so each copy reads whole row segments).
    // Chunk c of row r sits at slot c ^ mswz(r): a lane's 8-byte read of its row then
    // shares a bank pair with at most one other lane of its half-wave.
    i32x4 mrsrc = {0, 0, 0, 0};
    float ms2 = 0.f;  // slope * log2 e (softcap: scores in log2 units), else slope / scale (raw units)
    constexpr int MCH = BN * 2 / 16;       // 16-byte chunks per mask row of a tile
    constexpr int MRPI = 1024 / (BN * 2);  // mask rows per 1 KB copy
    auto mswz = [](int r) { return (r >> 1) & (MCH - 1); };
    char* const mstage = smem + 2 * STAGE + wave * MT;  // + stage * NW * MT
    if constexpr (ADDM) {
        const size_t slab = (size_t)p.Sq * (size_t)p.mask_stride;
        const uint16_t* mb = p.mask + ((size_t)(b % p.mask_batch) * p.mask_heads + (h % p.mask_heads)) * slab;
        mrsrc = make_buffer(mb, (uint32_t)(slab * 2));
        // ALiBi slope: m0^(h+1) below n_head_log2, else m1^(2(h - n_head_log2) + 1), with
        // m0 = 2^(-max_bias / n_head_log2) and m1 = 2^(-max_bias / (2 n_head_log2)); 1 when max_bias = 0
        const float e = h < p.n_head_log2 ? -(float)(h + 1) * p.max_bias / (float)p.n_head_log2
                                          : -(float)(2 * (h - p.n_head_log2) + 1) * p.max_bias /
                                                (2.f * (float)p.n_head_log2);
        ms2 = exp2_fast(e) * (SOFTCAP ? kLog2e : kLog2e / p.c_score);
    }
    // mask entries of tile t into stage st (keys past the slab end are not copied; they
    // only occur in the masked last tile, where those keys are excluded)
    auto mload = [&](int t, int st) {
        if constexpr (ADDM) {
#pragma unroll
            for (int j = 0; j < MT / 1024; ++j) {
                const int r = j * MRPI + lane / MCH;
                const int c = (lane % MCH) ^ mswz(r);
                const uint32_t off = (uint32_t)((size_t)min(q0 + r, p.Sq - 1) * (size_t)p.mask_stride * 2) +
                                     (uint32_t)(t * BN * 2 + c * 16);
                copy16(mrsrc, off, mstage + st * NW * MT + j * 1024);
            }
        }
    };
    if (ntiles > 0) mload(0, 0);
    // per-lane LDS byte offsets: K row col (both key blocks), 16-byte half `half`;
    // V^T rows half*4 + (lane&15)/4 of a 4-row transposing block, column
    // ((lane>>4)&1)*16 + (lane&3)*4 of a 32-column block
    const int kofs = col * 32 + ((half ^ ((col >> 3) & 1)) << 4);
    const int vofs = (half * 4 + ((lane & 15) >> 2)) * 64 + (((lane >> 4) & 1) * 16 + (lane & 3) * 4) * 2;

    auto tile = [&](const char* kt, const char* vt, const char* mt, int key0, auto mask_tag, auto&& post_qk) {
        constexpr bool MASK = decltype(mask_tag)::value;
        // S^T = K Q^T; K fragments are read from LDS PF steps ahead of their MFMA
        constexpr int NQK = KB * KK;
        constexpr int PFK = NQK < ATTN_PF_K ? NQK : ATTN_PF_K;
        auto kload = [&](int idx) -> bf16x8 {
            const int kb = idx / KK, kk = idx % KK;
            return *(const bf16x8*)(kt + kofs + kk * (BN * 32) + kb * 1024);
        };
        f32x16 sacc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
        bf16x8 kring[PFK];
#pragma unroll
        for (int i = 0; i < PFK; ++i) kring[i] = kload(i);
#pragma unroll
        for (int idx = 0; idx < NQK; ++idx) {
            const bf16x8 a = kring[idx % PFK];
            if (idx + PFK < NQK) kring[idx % PFK] = kload(idx + PFK);
            sacc[idx / KK] = mma32<F16>(a, qf[idx % KK], sacc[idx / KK]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (LATE) {
            post_qk();
            __builtin_amdgcn_sched_barrier(0);
        }
        // scores in log2 units (softcap) or raw (scaled inside the exponent), mask, tile max.
        // A softcapped tile with no mask of either kind takes its maximum over the raw scores
        // (the cap is increasing, so the capped maximum is the cap of the raw one) and keeps
        // only r = 1 / (e^{2y} + 1) per score: the exponent c_cap - 2 c_cap r - m is then one FMA.
        constexpr bool CAPR = SOFTCAP && !ADDM && !MASK;
        if constexpr (SOFTCAP && !CAPR) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    // cap * tanh(y), y = scale*x/cap, tanh(y) = 1 - 2 / (e^{2y} + 1), in log2 units
                    const float e = exp2_fast(sacc[kb][i] * p.c_tanh);
                    sacc[kb][i] = p.c_cap - 2.f * p.c_cap * __builtin_amdgcn_rcpf(e + 1.f);
                }
            }
        }
        if constexpr (ADDM) {
            // score plus slope * mask entry, in the score's units: log2 units after the softcap,
            // else raw, the scale joining the exponent as without a mask (fp16 -inf stays -inf)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const f16x4 mv = *(const f16x4*)(mt + col * (BN * 2) + (((kb * 4 + g4) ^ mswz(col)) << 4) + half * 8);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = g4 * 4 + e;
                        sacc[kb][i] = __builtin_fmaf((float)mv[e], ms2, sacc[kb][i]);
                    }
                }
            }
        }
        if constexpr (MASK) {  // diagonal and last tiles only
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = key0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
                    if (key > lim) sacc[kb][i] = -INFINITY;
                }
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        }
        mx = halfwave_max(mx);
        if constexpr (CAPR) mx = p.c_cap - 2.f * p.c_cap * __builtin_amdgcn_rcpf(exp2_fast(mx * p.c_tanh) + 1.f);
        const float cs = LOG2 ? 1.f : p.c_score;
        const float m_tile = LOG2 ? mx : mx * cs;
        // lazy reference update: only when the tile max exceeds the reference by > 2^tau
        const bool upd = m_tile > m_run + kTau;
        if (__builtin_amdgcn_ballot_w64(upd)) {
            // lanes that keep their reference (possibly still -inf) scale by exactly 1
            const float alpha = upd ? exp2_fast(m_run - m_tile) : 1.f;  // 0 when m_run = -inf
            m_run = upd ? m_tile : m_run;
            l_run *= alpha;
#pragma unroll
            for (int d = 0; d < DB; ++d) oacc[d] *= alpha;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        const float nm = -m_use;
        const float xa = CAPR ? -2.f * p.c_cap : cs, xb = CAPR ? p.c_cap + nm : nm;  // exponent xa * s + xb
        auto arg = [&](float x) { return CAPR ? __builtin_amdgcn_rcpf(exp2_fast(x * p.c_tanh) + 1.f) : x; };
        // P = 2^(s - m) rounded to bf16, packed as the PV operand; sum of the rounded values
        uint32_t pk[KB][8];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float p0 = exp2_fast(__builtin_fmaf(arg(sacc[kb][2 * j]), xa, xb));
                const float p1 = exp2_fast(__builtin_fmaf(arg(sacc[kb][2 * j + 1]), xa, xb));
                pk[kb][j] = pack_op2<F16>(p0, p1);
                l_run = add_op2<F16>(pk[kb][j], l_run);
            }
        }
        // O^T += V^T P^T, 16 keys per MFMA; V^T fragments read PF steps ahead
        constexpr int NPV = KB * 2 * DB;
        constexpr int PFV = NPV < ATTN_PF_V ? NPV : ATTN_PF_V;
        auto vload = [&](int idx) -> bf16x8 {
            const int d = idx % DB, jj = (idx / DB) % 2, kb = idx / (2 * DB);
            const char* pa = vt + vofs + d * (BN * 64) + kb * 2048 + jj * 1024;
            const bf16x4 va = lds_read_tr16(pa);
            const bf16x4 vb = lds_read_tr16(pa + 512);  // 8 rows further
            return __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8 vring[PFV];
#pragma unroll
        for (int i = 0; i < PFV; ++i) vring[i] = vload(i);
#pragma unroll
        for (int idx = 0; idx < NPV; ++idx) {
            const int d = idx % DB, jj = (idx / DB) % 2, kb = idx / (2 * DB);
            const bf16x8 a = vring[idx % PFV];
            if (idx + PFV < NPV) vring[idx % PFV] = vload(idx + PFV);
            const u32x4 pw = {pk[kb][4 * jj], pk[kb][4 * jj + 1], pk[kb][4 * jj + 2], pk[kb][4 * jj + 3]};
            oacc[d] = mma32<F16>(a, __builtin_bit_cast(bf16x8, pw), oacc[d]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Tiles [0, t_full) are visible to every row of the workgroup and run
    // without a mask; the rest (diagonal and ragged last tile) run masked.
    // Two separate loops keep each loop body one straight-line tile.
    int t_full = p.Sk / BN;
    if (CAUSAL) t_full = min(t_full, max(0, (qt * BM + shift + 1) / BN));
    t_full = min(t_full, ntiles);
    auto step = [&](int t) {
        wait_vmem();       // this wave's copies of tile t (K/V and its mask rows) have landed
        __syncthreads();   // ... and every other wave's; stage (t+1)&1 is free again
        if (!LATE && t + 1 < ntiles) {
            issue(t + 1, (t + 1) & 1);
            mload(t + 1, (t + 1) & 1);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto late = [&](int t) {  // LATE: the next tile's copies, issued after the QK product
        if (LATE && t + 1 < ntiles) {
            issue(t + 1, (t + 1) & 1);
            mload(t + 1, (t + 1) & 1);
        }
    };
#pragma clang loop unroll(disable)
    for (int t = 0; t < t_full; ++t) {
        step(t);
        const char* kt = smem + (t & 1) * STAGE;
        tile(kt, kt + K_BYTES, mstage + (t & 1) * NW * MT, t * BN, std::false_type{}, [&]() { late(t); });
    }
#pragma clang loop unroll(disable)
    for (int t = t_full; t < ntiles; ++t) {
        step(t);
        const char* kt = smem + (t & 1) * STAGE;
        const bool skip = CAUSAL && (t * BN > q0 + 31 + shift);  // wave-uniform
        if (!skip)
            tile(kt, kt + K_BYTES, mstage + (t & 1) * NW * MT, t * BN, std::true_type{}, [&]() { late(t); });
        else
            late(t);
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
        const size_t obase = (((size_t)b * p.Sq + qi) * p.Hq + h) * DV;
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

template <int DK, int DV, int BN, int NW, int OCC, bool CAUSAL, bool SOFTCAP, bool ADDM, bool F16>
hipError_t launch_variant(PrefillParams p, bool of32, hipStream_t stream) {
    constexpr int BM = NW * 32;
    p.nqt = (p.Sq + BM - 1) / BM;
    const dim3 grid((unsigned)(p.nqt * p.Hq * p.B)), block(NW * 64);
    if (of32)
        hipLaunchKernelGGL((prefill_kernel<DK, DV, BN, NW, OCC, CAUSAL, SOFTCAP, ADDM, F16, true>), grid, block, 0,
                           stream, p);
    else
        hipLaunchKernelGGL((prefill_kernel<DK, DV, BN, NW, OCC, CAUSAL, SOFTCAP, ADDM, F16, false>), grid, block, 0,
                           stream, p);
    return hipGetLastError();
}

template <int DK, int DV, int BN, int NW, int OCC, bool ADDM, bool F16>
hipError_t launch_flags(const PrefillParams& p, bool causal, bool softcap, bool of32, hipStream_t stream) {
    if (causal) {
        return softcap ? launch_variant<DK, DV, BN, NW, OCC, true, true, ADDM, F16>(p, of32, stream)
                       : launch_variant<DK, DV, BN, NW, OCC, true, false, ADDM, F16>(p, of32, stream);
    }
    return softcap ? launch_variant<DK, DV, BN, NW, OCC, false, true, ADDM, F16>(p, of32, stream)
                   : launch_variant<DK, DV, BN, NW, OCC, false, false, ADDM, F16>(p, of32, stream);
}

// (BN, NW, OCC) without a mask; (BNM, NWM, OCCM) with one
template <int DK, int DV, int BN, int NW, int OCC, int BNM = BN, int NWM = NW, int OCCM = OCC>
hipError_t launch_inst(const PrefillParams& p, bool kv_f16, bool causal, bool softcap, bool of32,
                       hipStream_t stream) {
    if (kv_f16) {
        if (p.mask != nullptr)
            return launch_flags<DK, DV, BNM, NWM, OCCM, true, true>(p, causal, softcap, of32, stream);
        return launch_flags<DK, DV, BN, NW, OCC, false, true>(p, causal, softcap, of32, stream);
    }
    if (p.mask != nullptr) return launch_flags<DK, DV, BNM, NWM, OCCM, true, false>(p, causal, softcap, of32, stream);
    return launch_flags<DK, DV, BN, NW, OCC, false, false>(p, causal, softcap, of32, stream);
}

// Kernel parameters from the launch arguments.
PrefillParams make_params(const PrefillArgs& a) {
    PrefillParams p;
    p.q = a.q;
    p.q_type = a.q_type;
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
    p.nqt = 0;
    p.c_score = a.scale * kLog2e;
    const bool softcap = a.softcap != 0.f;
    p.c_tanh = softcap ? 2.f * a.scale / a.softcap * kLog2e : 0.f;
    p.c_cap = a.softcap * kLog2e;
    p.xcd_remap = ((a.B * a.Hq) % 8) == 0;
    // grouped query heads per XCD: measured 3.5% faster for causal GQA at d=256. Without the
    // causal mask it was 2.4% slower while the tile copies were tracked; with the d = 256
    // unmasked kernel's copies issued untracked after the QK product it measured 1-2% faster
    // back to back (GQA 64:8, 4096^2: 865.6-877.9 against 874.5-894.5 us, same process, 8
    // rounds) and the same within 0.2% in the benchmark's sequence (894-896 us), so it applies
    // there too. Other head dims without the causal mask keep the heads spread (not measured).
    const bool late_copies = a.dk == 256 && a.dv == 256 && !a.causal && a.mask == nullptr;
    if ((a.causal || late_copies) && a.Hq != a.Hkv && ((a.B * a.Hkv) % 8) == 0) p.xcd_remap = 2;
    p.mask = (const uint16_t*)a.mask;
    p.mask_stride = a.mask_stride;
    p.mask_batch = a.mask_batch;
    p.mask_heads = a.mask_heads;
    p.max_bias = a.max_bias;
    int nl2 = 1;
    while (nl2 * 2 <= a.Hq) nl2 *= 2;
    p.n_head_log2 = nl2;
    return p;
}

}  // namespace

#ifdef ATTN_PREFILL_D256_UNIT
// Head dim 256 instances: a translation unit of their own, built with the max-ILP
// machine scheduler (measured 3% faster at GQA d=256, slower at d=128).
hipError_t launch_prefill_d256(const PrefillArgs& a, hipStream_t stream) {
    const PrefillParams p = make_params(a);
    return launch_inst<256, 256, ATTN_D256_CFG>(p, a.kv_f16 != 0, a.causal != 0, a.softcap != 0.f, a.o_f32 != 0,
                                                stream);
}
#else
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
    if (a.dk == 256 && a.dv == 256) return launch_prefill_d256(a, stream);
    const PrefillParams p = make_params(a);
    const bool of32 = a.o_f32 != 0, causal = a.causal != 0, kv_f16 = a.kv_f16 != 0, softcap = a.softcap != 0.f;
    switch (a.dk * 1000 + a.dv) {
        case 16016: return launch_inst<16, 16, 64, 4, 2>(p, kv_f16, causal, softcap, of32, stream);
        case 32032: return launch_inst<32, 32, 64, 4, 2>(p, kv_f16, causal, softcap, of32, stream);
        case 64064: return launch_inst<64, 64, 64, 4, 2>(p, kv_f16, causal, softcap, of32, stream);
        case 96096: return launch_inst<96, 96, 64, 4, 2>(p, kv_f16, causal, softcap, of32, stream);
        case 128128: return launch_inst<128, 128, ATTN_D128_CFG>(p, kv_f16, causal, softcap, of32, stream);
        // 64 keys x 8 waves without a mask (7-8% faster than 32 x 4 at B=2, H=32, 4096^2
        // causal); the masked instances keep 32 x 4
        case 192192: return launch_inst<192, 192, 64, 8, 2, 32, 4, 2>(p, kv_f16, causal, softcap, of32, stream);
        case 192128: return launch_inst<192, 128, 64, 8, 2, 32, 4, 2>(p, kv_f16, causal, softcap, of32, stream);
        default: return hipErrorInvalidValue;
    }
}
#endif

}  // namespace attn
