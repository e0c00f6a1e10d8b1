// Gathered-row decode attention (the MLA decode shape) for gfx950: the split-KV partial pass.
//
// Each token attends to its own list of rows of a row cache (the "MLA Decode
// Attention Kernel API Reference" page, Background and parameters: the selected
// prior rows are gathered straight from the cache in its native layout, no
// pre-gathered copy; a key is live iff its position is at or before the
// token's; the token's own row, kv_row_cur, is one more key, n_keys =
// n_prior + 1). The value is either a prefix of the key row (the page's latent
// is shared by key and value) or a row of a separate array with the same
// stride.
//
// Work: one workgroup per (token, group of 64 query heads, range of keys). Four
// waves, one per SIMD: waves w and w+2 own the same 32 heads (w & 1 picks the
// half) and take alternate 32-key steps of the range, so every gathered row is
// staged once for the workgroup and each wave sees half of them.
//   S^T [32 keys x 32 heads]  = K [32 x 576] Q^T         36 v_mfma_f32_32x32x16 per 32 keys
//   O^T [512 x 32 heads]     += V^T [512 x 32] P^T        32 v_mfma_f32_32x32x16 per 32 keys
// The 32x32x16 shape feeds 16K multiply-adds from every 1 KB fragment read out
// of LDS, twice the 16x16x32 shape's, and the 16 output blocks (256 registers
// per lane) live in the accumulation registers. A lane holds the scores of one
// head for 16 keys; the S^T accumulator is the P^T operand of the PV product
// after a round-to-nearest-even pack, with the keys of each 16-key half
// permuted to match, and V^T is read with ds_read_b64_tr_b16 in that order.
// At the end the two waves of a head pair merge their results through LDS
// (each takes half of the value columns) by the log-sum-exp identity.
//
// Sizing (the workload's 16 tokens x 128 heads x 2048 rows): 2 head groups x 8
// ranges of 256 keys per token give 256 workgroups. Each workgroup reads its
// 64 heads' queries (74 KB) and 256 rows (295 KB) and writes 64 KB of bf16
// partial output; with 128 heads per workgroup and 16 ranges the query
// re-reads and the partial output (147 + 128 KB per 147 KB of rows) made the
// pass bound by their traffic. All workgroups of a token are dispatched to one
// XCD (workgroup id % 8), so its L2 serves the token's queries and the rows its
// two head groups share.
//
// Rows are gathered 32 per step into four LDS stages (two steps computed while
// the next two are in flight) by direct HBM -> LDS copies, 1 KB per wave
// instruction. A stage is nine 4 KB blocks, block b holding 16-byte chunks
// 8b..8b+7 of the 32 rows at a 128-byte pitch: chunk c of row r sits at
// (c / 8) * 4096 + 128 r + 16 ((c % 8) ^ f(r)),
// f(r) = bit1(r) << 2 | (bit2(r) ^ bit3(r)) << 1 | bit3(r).
// Lane l of wave w copies row 8w + l/8 (its stored chunk l % 8 of every block), so
// a copy instruction fills 8 rows of one block and a lane looks up one row
// offset per step. The swizzle keeps both fragment reads free of bank conflicts:
//   K operand:   a 128-bit read by 32 consecutive rows x 2 adjacent chunks: any
//                16 consecutive rows at one chunk cover all 64 banks (with only
//                bits 1 and 2 of the row in f, rows r and r + 8 collided);
//   V^T operand: a transposing 64-bit read of 4 aligned rows x 4 chunks by 32
//                consecutive lanes.
// Each workgroup writes its range's output normalised by its own sum, rounded to
// bf16, with the fp32 running max (log2 units) and sum; the combine pass merges
// the ranges by log-sum-exp.
#include <type_traits>

#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {
namespace {

constexpr float kTauG = 8.f;  // lazy-rescale threshold (log2 units), as in the other kernels

struct GatherParams {
    const void* __restrict__ q;  // bf16, fp32 or fp16 (q_type)
    const uint16_t* __restrict__ kc;
    const uint16_t* __restrict__ vc;
    uint16_t* __restrict__ ws_o;  // [rows][n_split][DV] bf16: O_s / l_s
    float* __restrict__ ws_ml;    // [rows][n_split][2]: running max (log2 units), running sum
    const int32_t* __restrict__ row_index;
    const float* __restrict__ key_pos;
    const int32_t* __restrict__ q_pos;
    // token t's own key row at kc + kcur_off + t * row_stride, value row at vc + vcur_off + ...
    // (element offsets from the cache bases, so every gather address derives from one base pointer)
    long long kcur_off, vcur_off;
    int has_cur;
    int T, Hq, HG, n_sel, n_split, split_len;
    int xcd;  // 1: T is a multiple of 8 (every workgroup of a token on one XCD)
    long long row_stride;  // elements
    float c_score, c_tanh, c_cap;
    int q_type;
};

// chunk swizzle of stage row r (see the file comment)
__device__ __forceinline__ int gsw(int r) {
    return (((r >> 1) & 1) << 2) | ((((r >> 2) ^ (r >> 3)) & 1) << 1) | ((r >> 3) & 1);
}

// Direct HBM -> LDS copy of 16 bytes per lane (lane i writes lds + 16 i), written in assembly
// so that the compiler does not track it: tracked, it made the compiler wait for every copy in
// flight before some LDS reads of the stages being computed. The kernel orders each copy before
// the reads of its stage itself (a wait for the wave's copies, then a barrier). No output
// registers; M0 carries the LDS address.
__device__ __forceinline__ void dma16(const void* g, const void* lds) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(m) : "m0");
}

#ifndef ATTN_G_PFK
#define ATTN_G_PFK 4  // K fragments read ahead of their MFMA
#endif
#ifndef ATTN_G_PFV
#define ATTN_G_PFV 4  // V^T fragments read ahead of their MFMA
#endif

template <int DK, int DV, bool VK, bool F16, bool CAUSAL, bool SOFTCAP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void decode_gathered_kernel(GatherParams p) {
    constexpr int NW = 4, NT = 256;
    constexpr int KK = DK / 16;         // QK k-steps of 16
    constexpr int DB = DV / 32;         // 32-column blocks of O^T
    constexpr int DH = DB / 2;          // blocks each wave of a pair merges and stores
    constexpr int NCH = DK / 8;         // 16-byte chunks per key row
    constexpr int KBLK = NCH / 8;       // 4 KB blocks per key stage (8 chunks x 32 rows each)
    constexpr int VBLK = DV / 64;       // blocks holding the value columns
    constexpr int SSTAGE = KBLK * 4096; // one stage of 32 rows
    constexpr int STAGE = SSTAGE * (VK ? 1 : 2);
    constexpr int NST = VK ? 4 : 2;     // stages: two steps computed, (VK) two more in flight
    constexpr int IPT = (kGatherMaxSplit + NT - 1) / NT;  // table entries per thread
    static_assert(DK % 64 == 0 && DV % 64 == 0 && DV <= DK && NW * 8 == 32, "shape");
    static_assert(NST * STAGE + 12 * kGatherMaxSplit + 4 * IPT * NT / 32 <= 160 * 1024, "LDS");
    static_assert(NW * DH * 64 * 64 + NW * 64 * 8 <= NST * STAGE, "pair exchange fits the stages");
    __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];
    __shared__ long long skoff[kGatherMaxSplit];  // element offset of each key row from kc
    // key positions, +inf past the range's keys, -inf for every live key when not causal: a
    // key is live iff its entry is <= the token's position
    __shared__ __attribute__((aligned(16))) float spos[kGatherMaxSplit];
    __shared__ int slive[IPT * NT / 32];  // per 32-key step: all of its keys are live

    const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, col = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: copy destinations in SALU
    const int pair = wave & 1, par = wave >> 1;  // head half of the group; parity of the steps taken
    // workgroup -> (token, head group, key range). With xcd set, token t's workgroups run on
    // XCD t % 8 (workgroup id % 8), whose L2 then serves its queries and shared rows.
    const int per_tok = p.HG * p.n_split;
    int t, r;
    if (p.xcd) {
        const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
        t = x + 8 * (j / per_tok);
        r = j % per_tok;
    } else {
        t = blockIdx.x / per_tok;
        r = blockIdx.x % per_tok;
    }
    const int hg = r / p.n_split, split = r % p.n_split;
    const int start = split * p.split_len;
    const int end = min(p.n_sel, start + p.split_len);
    const int nsel = end - start;
    // the last range also takes the token's own row (n_keys = n_prior + 1), always live
    const int has_cur = (p.has_cur && split == p.n_split - 1) ? 1 : 0;
    const int nk = nsel + has_cur;
    const float qpos = (float)p.q_pos[t];

    // this range's row offsets and key positions (every load issued before the first LDS write)
    long long roff_r[IPT];
    float pos_r[IPT];
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
        const int i = tid + u * NT;
        roff_r[u] = 0;
        pos_r[u] = INFINITY;
        if (i < nsel) {
            roff_r[u] = (long long)p.row_index[(size_t)t * p.n_sel + start + i];
            pos_r[u] = CAUSAL ? p.key_pos[(size_t)t * p.n_sel + start + i] : -INFINITY;
        } else if (i == nsel && has_cur) {
            pos_r[u] = CAUSAL ? qpos : -INFINITY;
        }
    }
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
        const int i = tid + u * NT;
        if (i < nsel) skoff[i] = roff_r[u] * p.row_stride;
        if (i < kGatherMaxSplit) spos[i] = pos_r[u];
        // step (i / 32) is the lane's half of this wave: it needs no masking when every key is live
        const uint64_t b = __builtin_amdgcn_ballot_w64(pos_r[u] <= qpos);
        if (lane == 0) {
            const int s0 = (u * NT + wave * 64) >> 5;
            slive[s0] = (uint32_t)b == 0xffffffffu;
            slive[s0 + 1] = (uint32_t)(b >> 32) == 0xffffffffu;
        }
    }
    if (has_cur && tid == 0) skoff[nsel] = p.kcur_off + (long long)t * p.row_stride;
    __syncthreads();

    // Rows of step i into stage st: lane l of wave w copies row 8w + l/8 of the step, its
    // stored chunk l % 8 of every block (logical chunk 8b + ((l % 8) ^ f(row)) of block b), so
    // copy b of the wave writes bytes [1024 w, 1024 w + 1024) of block b. Rows past the range
    // repeat its last row, so every copy reads valid memory. Value rows (a separate array)
    // fill the blocks of a second stage the same way.
    const int crow = wave * 8 + (lane >> 3);
    const int cchunk = ((lane & 7) ^ gsw(crow)) * 8;  // element offset within a 64-element block
    auto issue = [&](int i, int st) {
        char* sb = smem + st * STAGE + wave * 1024;
        const int kr = min(i * 32 + crow, nk - 1);
        const long long ro = skoff[kr];
        const uint16_t* src = p.kc + ro + cchunk;
#pragma unroll
        for (int b = 0; b < KBLK; ++b) dma16(src + b * 64, sb + b * 4096);
        if constexpr (!VK) {
            const long long vo = ro + ((has_cur && kr == nsel) ? p.vcur_off - p.kcur_off : 0);
            const uint16_t* vsrc = p.vc + vo + cchunk;
#pragma unroll
            for (int b = 0; b < VBLK; ++b) dma16(vsrc + b * 64, sb + SSTAGE + b * 4096);
        }
    };
    const int nsteps = (nk + 31) / 32;
    if constexpr (VK) {
        issue(0, 0);
        if (nsteps > 1) issue(1, 1);
    }

    // per-lane LDS byte offsets within a stage (also used for the query rows below).
    // K operand of k-step kk = 4m + n: row col, logical chunk 2kk + hl = 8m + 2n + hl, in
    // block m at stored chunk (2n + hl) ^ f(col): kb[n] + 4096 m.
    int kb[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) kb[n] = col * 128 + (((2 * n + hl) ^ gsw(col)) << 4);

    // query fragments: head col of this pair's 32, dims kk*16 + hl*8 .. +7 (the B operand of
    // S^T = K Q^T). When Q already has the operand type, the group's 64 query rows are copied
    // into the two stages not yet in use (pair s's 32 rows into stage 2 + s, laid out and
    // copied like a step's key rows) and read back like K fragments; otherwise (Q converted
    // on load) each lane loads its 16-byte pieces.
    const int h = hg * 64 + pair * 32 + col;
    const bool hok = h < p.Hq;
    const bool wave_on = hg * 64 + pair * 32 < p.Hq;  // wave-uniform: any head of this wave exists
    bf16x8 qf[KK];
    const bool q_lds = VK && p.q_type == (F16 ? 2 : 0);
    if (q_lds) {
        char* qs = smem + 2 * STAGE;
        const uint16_t* qg = (const uint16_t*)p.q + ((size_t)t * p.Hq + hg * 64) * DK;
        const int qlast = min(64, p.Hq - hg * 64) - 1;  // rows past Hq repeat the last head
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const uint16_t* src = qg + (size_t)min(32 * s2 + crow, qlast) * DK + cchunk;
#pragma unroll
            for (int b = 0; b < KBLK; ++b) dma16(src + b * 64, qs + s2 * STAGE + wave * 1024 + b * 4096);
        }
        wait_vmem();
        __syncthreads();
        const char* qw = qs + pair * STAGE;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const bf16x8*)(qw + kb[kk & 3] + (kk >> 2) * 4096);
    } else {
        const size_t qrow = ((size_t)t * p.Hq + (hok ? h : 0)) * DK;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            qf[kk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
            if (hok) qf[kk] = load_q8<F16>(p.q, qrow + kk * 16 + hl * 8, p.q_type);
        }
    }

    // V^T operand of column block d, key half jj: two transposing reads of rows
    // 16 jj + 8 s + 4 hl + q (s = 0, 1; q = (lane & 15) / 4), columns d*32 + 16 bit4(lane) +
    // 4 (lane & 3) .. +3, i.e. logical chunk 4d + x with x = 2 bit4(lane) + bit1(lane): block
    // d >> 1, chunk 4 (d & 1) + x. f of those rows does not depend on jj, so the chunk is at
    // vb[d & 1][s] + 4096 (d >> 1) + 16 jj * 128.
    int vb[2][2];
    {
        const int q4 = (lane & 15) >> 2;
        const int x = (((lane >> 4) & 1) << 1) | ((lane >> 1) & 1);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int row = 8 * s2 + 4 * hl + q4;
                vb[b][s2] = row * 128 + (((4 * b + x) ^ gsw(row)) << 4) + ((lane & 1) << 3);
            }
    }

    // The 16 output blocks stay in the accumulation registers for the whole loop: the empty
    // asm statements with an accumulation-register operand pin them there at the loop edges
    // and around the (rare) rescale. Without the pins the compiler carried them across the
    // loop in ordinary registers, copying all 256 at every step and spilling ~1000 registers.
    f32x16 oacc[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) {
        oacc[d] = f32x16{};
        asm volatile("" : "+a"(oacc[d]));
    }
    float m_run = -INFINITY, l_run = 0.f;
    // The query fragments must have landed before the loop: otherwise the compiler, unable to
    // tell across the back edge whether their loads completed, waits for every outstanding
    // load (the next steps' row copies included) at their first use in every step.
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(qf[kk]));

#pragma clang loop unroll(disable)
    for (int i2 = 0; i2 < nsteps; i2 += 2) {
        if constexpr (!VK) {  // two stages of keys and values: load the pair, then compute it
            __syncthreads();  // every wave is done with the previous pair
            issue(i2, 0);
            if (i2 + 1 < nsteps) issue(i2 + 1, 1);
        }
        wait_vmem();      // this wave's copies of steps i2 and i2 + 1 landed
        __syncthreads();  // ... and every other wave's; the stages of steps i2 - 2, i2 - 1 are free
        if constexpr (VK) {
            if (i2 + 2 < nsteps) issue(i2 + 2, (i2 + 2) % NST);
            if (i2 + 3 < nsteps) issue(i2 + 3, (i2 + 3) % NST);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int i = i2 + par;  // this wave's step
        if (wave_on && i < nsteps) {
            const char* kt = smem + (i % NST) * STAGE;
            const char* vt = VK ? kt : kt + SSTAGE;
            const int r0 = i * 32;

            // S^T = K Q^T over the 36 k-steps, K fragments read PFK steps ahead. The MFMAs write
            // the accumulation registers, so the chain borrows one output block's (the compiler
            // parks that block in ordinary registers meanwhile); the first MFMA takes a literal
            // zero, and the scores move to ordinary registers once, for the softmax.
            constexpr int PFK = KK < ATTN_G_PFK ? KK : ATTN_G_PFK;
            auto kload = [&](int kk) -> bf16x8 { return *(const bf16x8*)(kt + kb[kk & 3] + (kk >> 2) * 4096); };
            f32x16 sacc;
            bf16x8 kring[PFK];
#pragma unroll
            for (int j = 0; j < PFK; ++j) kring[j] = kload(j);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const bf16x8 a = kring[kk % PFK];
                if (kk + PFK < KK) kring[kk % PFK] = kload(kk + PFK);
                sacc = mma32<F16>(a, qf[kk], kk == 0 ? f32x16{} : sacc);
                __builtin_amdgcn_sched_barrier(0);
            }
            asm volatile("" : "+v"(sacc));

            // masks and per-head maximum: lane value i3 is key r0 + 8 (i3 / 4) + 4 hl + i3 % 4 of
            // head col. Softcapped scores are transformed first (log2 units); plain ones stay raw
            // (the scale is positive, so the raw maximum gives the scaled one, and the scale
            // joins the exponent's fused multiply-add).
            if constexpr (SOFTCAP) {
#pragma unroll
                for (int i3 = 0; i3 < 16; ++i3) {
                    const float ex = exp2_fast(sacc[i3] * p.c_tanh);
                    sacc[i3] = p.c_cap - 2.f * p.c_cap * __builtin_amdgcn_rcpf(ex + 1.f);
                }
            }
            if (!__builtin_amdgcn_readfirstlane(slive[i])) {
                f32x4 kpos[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) kpos[j] = *(const f32x4*)(spos + r0 + 8 * j + 4 * hl);
#pragma unroll
                for (int i3 = 0; i3 < 16; ++i3)
                    if (!(kpos[i3 >> 2][i3 & 3] <= qpos)) sacc[i3] = -INFINITY;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int i3 = 0; i3 < 16; ++i3) mx = fmaxf(mx, sacc[i3]);
            mx = halfwave_max(mx);
            if constexpr (!SOFTCAP) mx *= p.c_score;  // -inf stays -inf
            const bool upd = mx > m_run + kTauG;
            const float alpha = upd ? exp2_fast(m_run - mx) : 1.f;  // 0 when m_run = -inf
            // the output of a lane whose reference was still -inf is zero: it needs no rescale
            // (without this test the first step of every wave rescaled all 256 accumulators)
            const bool rescale = __builtin_amdgcn_ballot_w64(upd && m_run != -INFINITY) != 0;
            m_run = upd ? mx : m_run;
            l_run *= alpha;
            if (rescale) {
#pragma unroll
                for (int d = 0; d < DB; ++d) {  // one block at a time
                    asm volatile("" : "+a"(oacc[d]));
                    oacc[d] *= alpha;
                    asm volatile("" : "+a"(oacc[d]));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            const float nm = (m_run == -INFINITY) ? 0.f : -m_run;
            uint32_t pk[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x0 = SOFTCAP ? sacc[2 * j] + nm : fmaf(sacc[2 * j], p.c_score, nm);
                const float x1 = SOFTCAP ? sacc[2 * j + 1] + nm : fmaf(sacc[2 * j + 1], p.c_score, nm);
                pk[j] = pack_op2<F16>(exp2_fast(x0), exp2_fast(x1));
                l_run = add_op2<F16>(pk[j], l_run);
            }

            // O^T += V^T P^T: 16 keys per MFMA, V^T fragments read PFV ahead
            constexpr int NPV = 2 * DB;
            constexpr int PFV = NPV < ATTN_G_PFV ? NPV : ATTN_G_PFV;
            const ATTN_LDS char* vtl = (const ATTN_LDS char*)vt;
            auto vload = [&](int idx) -> bf16x8 {
                const int jj = idx / DB, d = idx % DB;
                const int o = (d >> 1) * 4096 + (16 * jj) * 128;
                const bf16x4 va = lds_read_tr16_l(vtl + vb[d & 1][0] + o);
                const bf16x4 vv = lds_read_tr16_l(vtl + vb[d & 1][1] + o);
                return __builtin_shufflevector(va, vv, 0, 1, 2, 3, 4, 5, 6, 7);
            };
            bf16x8 vring[PFV];
#pragma unroll
            for (int j = 0; j < PFV; ++j) vring[j] = vload(j);
#pragma unroll
            for (int idx = 0; idx < NPV; ++idx) {
                const int jj = idx / DB, d = idx % DB;
                const bf16x8 a = vring[idx % PFV];
                if (idx + PFV < NPV) vring[idx % PFV] = vload(idx + PFV);
                const u32x4 pw = {pk[4 * jj], pk[4 * jj + 1], pk[4 * jj + 2], pk[4 * jj + 3]};
                oacc[d] = mma32<F16>(a, __builtin_bit_cast(bf16x8, pw), oacc[d]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int d = 0; d < DB; ++d) asm volatile("" : "+a"(oacc[d]));
    }

    // Merge the two waves of each head pair through LDS (the stages are free once every wave
    // is past its last step): the even-step wave keeps value columns [0, DV/2) and hands the
    // rest to its partner, the odd-step wave the other way round. An exchanged block is stored
    // as 4 slices of 4 accumulators, each slice 16 contiguous bytes per lane (1 KB per read or
    // write, no bank conflicts), so partner lane l reads exactly its own elements.
    const float l_tot = halfwave_sum(l_run);
    __syncthreads();
    float* xo = (float*)smem;                     // [wave][DH blocks][4 slices][64 lanes][4]
    float* xml = (float*)(smem + NW * DH * 4096);  // [wave][64 lanes][2]
    // (block offsets are compile-time constants in each branch: a run-time index into the
    // accumulator array would place the whole array in scratch memory)
    auto give = [&](auto g0) {
        constexpr int G0 = decltype(g0)::value;
#pragma unroll
        for (int d = 0; d < DH; ++d) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                *(f32x4*)(xo + (((wave * DH + d) * 4 + c) * 64 + lane) * 4) =
                    f32x4{oacc[G0 + d][4 * c], oacc[G0 + d][4 * c + 1], oacc[G0 + d][4 * c + 2],
                          oacc[G0 + d][4 * c + 3]};
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (par)
        give(std::integral_constant<int, 0>{});
    else
        give(std::integral_constant<int, DH>{});
    xml[(wave * 64 + lane) * 2] = m_run;
    xml[(wave * 64 + lane) * 2 + 1] = l_tot;
    __syncthreads();
    const int partner = wave ^ 2;
    const float mp = xml[(partner * 64 + lane) * 2], lp = xml[(partner * 64 + lane) * 2 + 1];
    const float M = fmaxf(m_run, mp);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    const float fa = exp2_fast(m_run - Mu), fb = exp2_fast(mp - Mu);  // 2^-inf = 0
    const float l_sum = l_tot * fa + lp * fb;
    const float inv = l_sum > 0.f ? 1.f / l_sum : 0.f;
    const float ca = fa * inv, cb = fb * inv;
    if (hok && hl == 0 && par == 0) {
        const size_t slot = ((size_t)t * p.Hq + h) * p.n_split + split;
        p.ws_ml[slot * 2] = M;
        p.ws_ml[slot * 2 + 1] = l_sum;
    }
    // merged, normalised columns of this wave's half, rounded to bf16 (lane value i of block d
    // is column d*32 + 8 (i / 4) + 4 hl + i % 4 of head col)
    u32x2 outp[DH][4];
    auto keep = [&](auto k0) {
        constexpr int K0 = decltype(k0)::value;
#pragma unroll
        for (int d = 0; d < DH; ++d) {
            asm volatile("" : "+a"(oacc[K0 + d]));
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f32x4 o = *(const f32x4*)(xo + (((partner * DH + d) * 4 + c) * 64 + lane) * 4);
                outp[d][c] = u32x2{pack_bf16x2(oacc[K0 + d][4 * c] * ca + o[0] * cb,
                                               oacc[K0 + d][4 * c + 1] * ca + o[1] * cb),
                                   pack_bf16x2(oacc[K0 + d][4 * c + 2] * ca + o[2] * cb,
                                               oacc[K0 + d][4 * c + 3] * ca + o[3] * cb)};
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (par)
        keep(std::integral_constant<int, DH>{});
    else
        keep(std::integral_constant<int, 0>{});
    __syncthreads();  // every wave has read its partner's blocks: the exchange area is free
    // staging [pair][32 heads][DV] bf16 (a 16-byte pad per row), then whole 1 KB rows out.
    // Rows 16-31 hold the two 8-byte halves of every 16-byte chunk swapped: then the 8-byte
    // writes of rows r and r + 16 (1040 bytes apart per row) fall in different banks.
    constexpr int OPITCH = DV * 2 + 16;
    static_assert(2 * 32 * OPITCH <= NST * STAGE, "output staging fits the stages");
    char* ost = smem + pair * 32 * OPITCH;
    const int keep0 = par ? DH : 0;
    char* ow = ost + col * OPITCH + 8 * (hl ^ (col >> 4));
#pragma unroll
    for (int d = 0; d < DH; ++d)
#pragma unroll
        for (int c = 0; c < 4; ++c) *(u32x2*)(ow + ((keep0 + d) * 32 + 8 * c) * 2) = outp[d][c];
    __syncthreads();
    // each wave stores 16 of its pair's 32 head rows (the odd-step wave rows 16-31, which it
    // swaps back), 1 KB per instruction
    constexpr int PER = DV * 2 / 1024;
    auto store_rows = [&](auto sw) {
        constexpr bool SW = decltype(sw)::value;
#pragma unroll 4
        for (int k = 0; k < 16 * PER; ++k) {
            const int hh = (SW ? 16 : 0) + k / PER, part = k % PER;
            const int head = hg * 64 + pair * 32 + hh;
            if (head < p.Hq) {
                const size_t slot = ((size_t)t * p.Hq + head) * p.n_split + split;
                const u32x4 v = *(const u32x4*)(ost + hh * OPITCH + part * 1024 + lane * 16);
                __builtin_nontemporal_store(SW ? u32x4{v[2], v[3], v[0], v[1]} : v,
                                            (u32x4*)((char*)p.ws_o + slot * (DV * 2) + part * 1024 + lane * 16));
            }
        }
    };
    if (par)
        store_rows(std::true_type{});
    else
        store_rows(std::false_type{});
}

template <bool VK, bool F16, bool CAUSAL, bool SOFTCAP>
hipError_t launch_t(const GatherParams& gp, unsigned nwg, hipStream_t stream) {
    hipLaunchKernelGGL((decode_gathered_kernel<576, 512, VK, F16, CAUSAL, SOFTCAP>), dim3(nwg), dim3(256), 0, stream,
                       gp);
    return hipGetLastError();
}
template <bool VK, bool F16>
hipError_t launch_f(const GatherParams& gp, bool causal, bool softcap, unsigned nwg, hipStream_t stream) {
    if (causal)
        return softcap ? launch_t<VK, F16, true, true>(gp, nwg, stream) : launch_t<VK, F16, true, false>(gp, nwg, stream);
    return softcap ? launch_t<VK, F16, false, true>(gp, nwg, stream) : launch_t<VK, F16, false, false>(gp, nwg, stream);
}

}  // namespace

int gathered_head_groups(int Hq) { return (Hq + 63) / 64; }

hipError_t launch_gathered_split(const DecodeArgs& a, const DecodePlan& pl, uint16_t* ws_o, float* ws_ml,
                                 hipStream_t stream) {
    GatherParams gp;
    gp.q = a.q;
    gp.q_type = a.q_type;
    gp.kc = (const uint16_t*)a.k_cache;
    gp.vc = (const uint16_t*)a.v_cache;
    gp.ws_o = ws_o;
    gp.ws_ml = ws_ml;
    gp.row_index = a.row_index;
    gp.key_pos = a.key_pos;
    gp.q_pos = a.q_pos;
    gp.has_cur = a.k_cur != nullptr;
    gp.kcur_off = gp.has_cur ? (long long)((const uint16_t*)a.k_cur - (const uint16_t*)a.k_cache) : 0;
    gp.vcur_off = gp.has_cur ? (long long)((const uint16_t*)a.v_cur - (const uint16_t*)a.v_cache) : 0;
    gp.T = a.B;
    gp.Hq = a.Hq;
    gp.HG = gathered_head_groups(a.Hq);
    gp.n_sel = a.n_sel;
    gp.n_split = pl.n_split;
    gp.split_len = pl.split_len;
    gp.row_stride = a.row_stride;
    const bool softcap = a.softcap != 0.f;
    gp.c_score = a.scale * kLog2e;
    gp.c_tanh = softcap ? 2.f * a.scale / a.softcap * kLog2e : 0.f;
    gp.c_cap = a.softcap * kLog2e;
    gp.xcd = (a.B % 8) == 0;
    const unsigned nwg = (unsigned)((long long)a.B * gp.HG * pl.n_split);
    const bool vk = a.v_cache == a.k_cache, f16 = a.kv_f16 != 0, causal = a.causal != 0;
    if (vk)
        return f16 ? launch_f<true, true>(gp, causal, softcap, nwg, stream)
                   : launch_f<true, false>(gp, causal, softcap, nwg, stream);
    return f16 ? launch_f<false, true>(gp, causal, softcap, nwg, stream)
               : launch_f<false, false>(gp, causal, softcap, nwg, stream);
}

}  // namespace attn
