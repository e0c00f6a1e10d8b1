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
// instruction. Stage rows sit at the row pitch (1152 bytes, 128 mod 256) with
// 16-byte chunk c of row r stored at c ^ f(r), f(r) = bit1(r) << 2 | bit2(r) << 1,
// which keeps both fragment reads free of bank conflicts:
//   K operand:   a 128-bit read by 32 consecutive rows x 2 adjacent chunks
//                (the LDS serves lanes 0-7 with 32-39, rows 8m..8m+7);
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
__device__ __forceinline__ int gsw(int r) { return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1); }

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
    constexpr int PITCH = DK * 2;       // LDS row pitch (bytes), key and value stages alike
    constexpr int NCH = DK / 8;         // 16-byte chunks per row
    constexpr int SSTAGE = 32 * PITCH;  // one stage of 32 rows
    constexpr int NSEG = SSTAGE / 1024; // 1 KB direct loads per stage
    constexpr int STAGE = SSTAGE * (VK ? 1 : 2);
    constexpr int NST = VK ? 4 : 2;     // stages: two steps computed, (VK) two more in flight
    constexpr int JW = NSEG / NW;       // copies per wave per stage (key rows)
    static_assert(DK % 32 == 0 && DV % 64 == 0 && DV <= DK && PITCH % 256 == 128, "shape");
    static_assert(SSTAGE % 1024 == 0 && NSEG % NW == 0 && NCH % 8 == 0, "stage");
    static_assert(NST * STAGE + 12 * kGatherMaxSplit <= 160 * 1024, "LDS");
    static_assert(NW * DH * 64 * 64 + NW * 64 * 8 <= NST * STAGE, "pair exchange fits the stages");
    __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];
    __shared__ long long skoff[kGatherMaxSplit];  // element offset of each key row from kc
    __shared__ __attribute__((aligned(16))) float spos[kGatherMaxSplit];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hl = lane >> 5, col = lane & 31;
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

    // this range's row indices and positions (every load issued before the first LDS write)
    constexpr int IPT = (kGatherMaxSplit + NT - 1) / NT;
    long long roff_r[IPT];
    float pos_r[IPT];
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
        const int i = tid + u * NT;
        roff_r[u] = 0;
        pos_r[u] = 0.f;
        if (i < nsel) {
            roff_r[u] = (long long)p.row_index[(size_t)t * p.n_sel + start + i];
            if (CAUSAL) pos_r[u] = p.key_pos[(size_t)t * p.n_sel + start + i];
        }
    }
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
        const int i = tid + u * NT;
        if (i < nsel) {
            skoff[i] = roff_r[u] * p.row_stride;
            spos[i] = pos_r[u];
        }
    }
    if (has_cur && tid == 0) {
        skoff[nsel] = p.kcur_off + (long long)t * p.row_stride;
        spos[nsel] = qpos;
    }
    __syncthreads();

    // Rows of step i into stage st: wave w fills 1 KB segments w, w+NW, ... All row offsets
    // of the step are read from LDS before the first copy is issued (a copy writes LDS, so a
    // later table read could not be moved ahead of it). Rows past the range repeat its last
    // row, so every copy reads valid memory.
    auto issue = [&](int i, int st) {
        char* sb = smem + st * STAGE;
        if constexpr (!VK) {
            // separate value rows: twice the copies; issued one row at a time, which keeps the
            // register peak low (all offsets first made this variant spill)
#pragma unroll 1
            for (int j = 0; j < JW; ++j) {
                const int sg = wave + j * NW;
                const int off = sg * 1024 + lane * 16;
                const int rr = off / PITCH;
                const int kr1 = min(i * 32 + rr, nk - 1);
                const long long ro1 = skoff[kr1];
                const int c = ((off - rr * PITCH) >> 4) ^ gsw(rr);
                load_lds16(p.kc + ro1 + c * 8, sb + sg * 1024);
                // value rows use the same layout; chunks past the value width repeat earlier ones
                const long long vo = ro1 + ((has_cur && kr1 == nsel) ? p.vcur_off - p.kcur_off : 0);
                load_lds16(p.vc + vo + (c % (DV / 8)) * 8, sb + SSTAGE + sg * 1024);
            }
            return;
        }
        long long ro[JW];
        int kr[JW];
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const int rr = ((wave + j * NW) * 1024 + lane * 16) / PITCH;
            kr[j] = min(i * 32 + rr, nk - 1);
            ro[j] = skoff[kr[j]];
        }
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const int sg = wave + j * NW;
            const int off = sg * 1024 + lane * 16;
            const int rr = off / PITCH;
            const int c = ((off - rr * PITCH) >> 4) ^ gsw(rr);
            load_lds16(p.kc + ro[j] + c * 8, sb + sg * 1024);
        }
    };
    const int nsteps = (nk + 31) / 32;
    if constexpr (VK) {
        issue(0, 0);
        if (nsteps > 1) issue(1, 1);
    }

    // per-lane LDS byte offsets within a stage (also used for the query rows below).
    // K operand of k-step kk: row col, logical chunk 2kk + hl, stored at (2kk + hl) ^ f(col)
    //   = 2 (kk ^ g) + hl with g = f(col) / 2; for kk = 4m + n that is kb[n] + 128 m.
    int kb[4];
    {
        const int g = gsw(col) >> 1;
#pragma unroll
        for (int n = 0; n < 4; ++n) kb[n] = col * PITCH + ((n ^ g) << 5) + (hl << 4);
    }

    // query fragments: head col of this pair's 32, dims kk*16 + hl*8 .. +7 (the B operand of
    // S^T = K Q^T). When Q already has the operand type, the group's 64 query rows (contiguous
    // in memory, 64 * DK * 2 bytes = two stages) are copied into the two stages not yet in
    // use with whole 1 KB loads and read back like K fragments; otherwise (Q converted on
    // load) each lane loads its 16-byte pieces.
    const int h = hg * 64 + pair * 32 + col;
    const bool hok = h < p.Hq;
    const bool wave_on = hg * 64 + pair * 32 < p.Hq;  // wave-uniform: any head of this wave exists
    bf16x8 qf[KK];
    const bool q_lds = VK && p.q_type == (F16 ? 2 : 0);
    if (q_lds) {
        static_assert(64 * PITCH <= 2 * STAGE, "query rows fit two stages");
        char* qs = smem + 2 * STAGE;
        const uint16_t* qg = (const uint16_t*)p.q + ((size_t)t * p.Hq + hg * 64) * DK;
        const int qlast = min(64, p.Hq - hg * 64) - 1;  // rows past Hq repeat the last head
        constexpr int QSEG = 64 * PITCH / 1024;
#pragma unroll
        for (int j = 0; j < QSEG / NW; ++j) {
            const int sg = wave + j * NW;
            const int off = sg * 1024 + lane * 16;
            const int rr = off / PITCH;
            const int c = ((off - rr * PITCH) >> 4) ^ gsw(rr);
            load_lds16(qg + (size_t)min(rr, qlast) * DK + c * 8, qs + sg * 1024);
        }
        wait_vmem();
        __syncthreads();
        const char* qw = qs + pair * 32 * PITCH;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const bf16x8*)(qw + kb[kk & 3] + (kk >> 2) * 128);
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
    // 4 (lane & 3) .. +3, i.e. logical chunk 4d + x with x = 2 bit4(lane) + bit1(lane).
    // f of those rows is a << 2 | hl << 1 (a = bit1(q)), so the chunk is stored at
    // 4 (d ^ a) + (x ^ 2 hl): vb[d & 1] + 128 (d >> 1) + (16 jj + 8 s) * PITCH.
    int vb[2];
    {
        const int q4 = (lane & 15) >> 2, a = (q4 >> 1) & 1;
        const int x = (((lane >> 4) & 1) << 1) | ((lane >> 1) & 1);
#pragma unroll
        for (int b = 0; b < 2; ++b)
            vb[b] = (4 * hl + q4) * PITCH + ((b ^ a) << 6) + ((x ^ (hl << 1)) << 4) + ((lane & 1) << 3);
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
            auto kload = [&](int kk) -> bf16x8 { return *(const bf16x8*)(kt + kb[kk & 3] + (kk >> 2) * 128); };
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

            // scores (log2 units), masks, per-head maximum: lane value i3 is key
            // r0 + 8 (i3 / 4) + 4 hl + i3 % 4 of head col
            f32x4 kpos[4];
            if constexpr (CAUSAL) {
#pragma unroll
                for (int j = 0; j < 4; ++j) kpos[j] = *(const f32x4*)(spos + r0 + 8 * j + 4 * hl);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int i3 = 0; i3 < 16; ++i3) {
                float x = sacc[i3];
                if constexpr (SOFTCAP) {
                    const float ex = exp2_fast(x * p.c_tanh);
                    x = p.c_cap - 2.f * p.c_cap * __builtin_amdgcn_rcpf(ex + 1.f);
                } else {
                    x *= p.c_score;
                }
                const int kl = r0 + 8 * (i3 >> 2) + 4 * hl + (i3 & 3);
                bool live = kl < nk;
                if constexpr (CAUSAL) live = live && kpos[i3 >> 2][i3 & 3] <= qpos;
                if (!live) x = -INFINITY;
                sacc[i3] = x;
                mx = fmaxf(mx, x);
            }
            mx = halfwave_max(mx);
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
                pk[j] = pack_op2<F16>(exp2_fast(sacc[2 * j] + nm), exp2_fast(sacc[2 * j + 1] + nm));
                l_run = add_op2<F16>(pk[j], l_run);
            }

            // O^T += V^T P^T: 16 keys per MFMA, V^T fragments read PFV ahead
            constexpr int NPV = 2 * DB;
            constexpr int PFV = NPV < ATTN_G_PFV ? NPV : ATTN_G_PFV;
            const ATTN_LDS char* vtl = (const ATTN_LDS char*)vt;
            auto vload = [&](int idx) -> bf16x8 {
                const int jj = idx / DB, d = idx % DB;
                const ATTN_LDS char* pa = vtl + vb[d & 1] + (d >> 1) * 128 + (16 * jj) * PITCH;
                const bf16x4 va = lds_read_tr16_l(pa);
                const bf16x4 vv = lds_read_tr16_l(pa + 8 * PITCH);
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
    // staging [pair][32 heads][DV] bf16 (a 16-byte pad per row), then whole 1 KB rows out
    constexpr int OPITCH = DV * 2 + 16;
    static_assert(2 * 32 * OPITCH <= NST * STAGE, "output staging fits the stages");
    char* ost = smem + pair * 32 * OPITCH;
    const int keep0 = par ? DH : 0;
#pragma unroll
    for (int d = 0; d < DH; ++d)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *(u32x2*)(ost + col * OPITCH + ((keep0 + d) * 32 + 8 * c + 4 * hl) * 2) = outp[d][c];
    __syncthreads();
    // each wave stores 16 of its pair's 32 head rows, 1 KB per instruction
    constexpr int PER = DV * 2 / 1024;
#pragma unroll 4
    for (int k = 0; k < 16 * PER; ++k) {
        const int hh = par * 16 + k / PER, part = k % PER;
        const int head = hg * 64 + pair * 32 + hh;
        if (head < p.Hq) {
            const size_t slot = ((size_t)t * p.Hq + head) * p.n_split + split;
            *(u32x4*)((char*)p.ws_o + slot * (DV * 2) + part * 1024 + lane * 16) =
                *(const u32x4*)(ost + hh * OPITCH + part * 1024 + lane * 16);
        }
    }
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
