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
#include <mutex>

#include "attn_device.hpp"
#include "attn_launch.hpp"

// Split-KV scratch of the no-allocation decode entry point: one copy per GPU, held for the
// life of the process. In host code this name is only a stand-in for the symbol: kernels
// and copies take the device address that noalloc_scratch() looks up, never this name.
static __device__ __align__(256) char scratch[attn::kNoallocScratchBytes];

namespace attn {
namespace {

struct SplitParams {
    const void* __restrict__ q;  // bf16, fp32 or fp16 (q_type)
    const uint16_t* __restrict__ kc;
    const uint16_t* __restrict__ vc;
    float* __restrict__ ws_o;   // [rows][n_split][dv]
    float* __restrict__ ws_ml;  // [rows][n_split][2]
    const int32_t* __restrict__ block_table;
    const int32_t* __restrict__ seq_lens;
    int B, Hq, Hkv, Sq, group, nq, bs_log2, max_blocks;
    int ncg;  // groups of 16 * CB query columns per KV head (one workgroup each)
    int n_split, split_len;
    float c_score, c_tanh, c_cap;
    int causal, softcap_on;
    int q_type;  // 0 bf16, 1 fp32, 2 fp16
};

constexpr float kTau = 8.f;  // lazy-rescale threshold (log2 units), as in the prefill kernel

// One wavefront per (split, KV head, sequence). 32 keys per step on
// 16x16x32 MFMA: S^T[16 keys x 16 query columns] blocks, so a lane holds 4
// keys of one query column per block; up to CB blocks of 16 query columns.
// K fragments go HBM -> registers one step ahead; V rows go HBM -> LDS (one
// 1 KB direct load per instruction) one step ahead into a per-wave double
// buffer, for the transposing read of the V^T operand.
// F16: the caches (and the MFMA operands, P included) are IEEE fp16 instead of bf16.
template <int DK, int DV, int CB, bool F16>
// head dims <= 128 aim for two waves per SIMD (4% faster with 32 query columns; larger dims
// would spill), larger ones for one
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(DK <= 128 ? 2 : 1)))
void decode_paged_split_kernel(SplitParams p) {
    constexpr int DKP = DK < 32 ? 32 : DK;  // QK k-steps of 32 (zero-padded)
    constexpr int KQ = DKP / 32;
    constexpr int DBV = DV / 16;            // 16-row blocks of O^T
    constexpr int NCV = DV / 8;             // 16-byte chunks per V row
    constexpr int VROW = DV * 2;            // bytes per V row
    constexpr int STAGE = 32 * VROW;        // one step of V
    constexpr int VSEG = STAGE / 1024;      // 1 KB direct-load instructions per step
    static_assert(STAGE % 1024 == 0, "V step must split into 1 KB segments");
    __shared__ __attribute__((aligned(1024))) char vl[2 * STAGE];

    const int lane = threadIdx.x, grp = lane >> 4, c16 = lane & 15;
    // split-major grid: every (KV head, sequence) pair of split 0 first, then split 1, ...,
    // so the last work dispatched belongs to the longest sequences' final (often partial) splits
    const int split = blockIdx.z, g = blockIdx.x / p.ncg, cg0 = (blockIdx.x % p.ncg) * (16 * CB), b = blockIdx.y;
    const int L = p.seq_lens[b];
    const int start = split * p.split_len;
    if (start >= L) return;  // the combine pass only reads splits that start below L
    const int end = min(L, start + p.split_len);
    const int bs = 1 << p.bs_log2;
    const int32_t* table = p.block_table + (size_t)b * p.max_blocks;

    // keep LDS finite everywhere; the zeros must land before any direct load writes LDS
    for (int i = lane; i < 2 * STAGE / 16; i += 64) *(u32x4*)(vl + i * 16) = u32x4{0, 0, 0, 0};
    __syncthreads();

    // query columns cb*16 + c16 -> (query row, head of this KV group)
    bf16x8 qf[CB][KQ];
    int lim[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int colq = cg0 + cb * 16 + c16;
        const bool ok = colq < p.nq;
        const int si = ok ? colq / p.group : 0;
        const int h = g * p.group + (ok ? colq % p.group : 0);
        const size_t qrow = (((size_t)b * p.Sq + si) * p.Hq + h) * DK;
#pragma unroll
        for (int kk = 0; kk < KQ; ++kk) {
            const int dk0 = kk * 32 + grp * 8;
            qf[cb][kk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
            if (ok && dk0 < DK) qf[cb][kk] = load_q8<F16>(p.q, qrow + dk0, p.q_type);
        }
        lim[cb] = min(end - 1, p.causal ? L - p.Sq + si : L - 1);  // last key this column may see
    }

    // A 32-key step (32-aligned) lies in at most two cache blocks; their table
    // entries are read with wave-uniform (scalar) loads so that only K and V
    // loads sit in the vector-memory queue. Keys past L are clamped to L - 1
    // (in the same step) so every load is issued and reads finite data.
    const int lastb = (L - 1) >> p.bs_log2;
    const __attribute__((address_space(4))) int32_t* ctable =
        (const __attribute__((address_space(4))) int32_t*)table;  // read-only: scalar loads
    auto step_blocks = [&](int k0, int& blkA, int& blkB) {
        blkA = ctable[k0 >> p.bs_log2];
        blkB = ctable[min((k0 + 16) >> p.bs_log2, lastb)];
    };
    auto row_off = [&](int k0, int key, int blkA, int blkB) -> size_t {
        key = min(key, L - 1);
        const int blk = (key - k0) < 16 ? blkA : blkB;
        return ((size_t)blk * p.Hkv + g) * bs + (key & (bs - 1));
    };
    // Keys k0..k0+15 lie in block blkA and k0+16..k0+31 in blkB (k0 is a multiple of 32, blocks
    // hold >= 16 keys, and a key clamped to L - 1 stays in its half's block). A K fragment row
    // (kb*16 + c16), and a V segment when 16 rows fill whole 1 KB segments, therefore read one
    // block: a wave-uniform (scalar) block base plus a 32-bit per-lane offset inside the block.
    // The 32-column instance addresses this way: with 64-bit per-lane addresses it spilled 13
    // registers, and each reload's full vector-memory wait also waited for the next step's
    // loads (4 tokens x 8 heads at config 4: 1027 -> 978 us). The 16-column instances keep
    // per-lane addresses, 3-4% faster at d = 128 and 192/128 on 1024..8192-key sequences.
    constexpr bool SBASE = CB == 2;
    auto kv_base = [&](const uint16_t* cache, int blk, int d) -> const char* {
        return (const char*)(cache + ((size_t)blk * p.Hkv + g) * bs * d);
    };
    auto row_in_block = [&](int key) -> uint32_t { return (uint32_t)(min(key, L - 1) & (bs - 1)); };
    // K fragments of step k0: block kb, k-step kk: key k0 + kb*16 + c16, dk kk*32 + grp*8
    auto kload = [&](int k0, int blkA, int blkB, u32x4 (&kr)[2][KQ]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if constexpr (SBASE) {
                const char* base = kv_base(p.kc, kb ? blkB : blkA, DK);
                const uint32_t ro = row_in_block(k0 + kb * 16 + c16) * (DK * 2);  // bytes
#pragma unroll
                for (int kk = 0; kk < KQ; ++kk) {
                    const int dk0 = kk * 32 + grp * 8;
                    if (dk0 < DK)
                        kr[kb][kk] = *(const u32x4*)(base + (size_t)(ro + (uint32_t)(dk0 * 2)));
                    else
                        kr[kb][kk] = u32x4{0, 0, 0, 0};
                }
            } else {
                const uint16_t* r = p.kc + row_off(k0, k0 + kb * 16 + c16, blkA, blkB) * DK;
#pragma unroll
                for (int kk = 0; kk < KQ; ++kk) {
                    const int dk0 = kk * 32 + grp * 8;
                    if (dk0 < DK)
                        kr[kb][kk] = *(const u32x4*)(r + dk0);
                    else
                        kr[kb][kk] = u32x4{0, 0, 0, 0};
                }
            }
        }
    };
    // V rows of step k0 into stage st (swizzled 16-byte chunks), non-temporal: each row is read
    // once (measured 9% faster at 64 sequences of up to 32K keys; the same hint on K was slower)
    auto vload = [&](int k0, int blkA, int blkB, int st) {
#pragma unroll
        for (int s = 0; s < VSEG; ++s) {
            const int off = s * 1024 + lane * 16;
            const int r = off / VROW;
            const int c = ((off % VROW) >> 4) ^ swz<NCV, true>(r);
            if constexpr (SBASE && (16 * VROW) % 1024 == 0) {
                const char* base = kv_base(p.vc, s >= 16 * VROW / 1024 ? blkB : blkA, DV);
                load_lds16_nt(base + (size_t)(row_in_block(k0 + r) * (DV * 2) + (uint32_t)(c * 16)),
                              vl + st * STAGE + s * 1024);
            } else {
                load_lds16_nt(p.vc + row_off(k0, k0 + r, blkA, blkB) * DV + c * 8, vl + st * STAGE + s * 1024);
            }
        }
    };

    f32x4 oacc[CB][DBV];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int d = 0; d < DBV; ++d) oacc[cb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[CB], l_run[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        m_run[cb] = -INFINITY;
        l_run[cb] = 0.f;
    }

    // one 32-key step: S^T, online softmax, O^T += V^T P^T (K fragments in kc_, V in stage st)
    // V^T fragments of stage st into registers: for column block d, rows (keys) grp*4 + 0..3 of
    // block 0 and 16 + grp*4 + 0..3 of block 1, columns d*16 + (c16&3)*4 + 0..3
    auto vread = [&](int st, bf16x8 (&vf)[DBV]) {
        const char* vt = vl + st * STAGE;
        const int ra = grp * 4 + (c16 >> 2);
        const int rb = ra + 16;
#pragma unroll
        for (int d = 0; d < DBV; ++d) {
            const int dc = d * 16 + (c16 & 3) * 4;
            const int ch = dc >> 3, within = (dc & 7) * 2;
            const bf16x4 va = lds_read_tr16(vt + ra * VROW + ((ch ^ swz<NCV, true>(ra)) * 16) + within);
            const bf16x4 vb = lds_read_tr16(vt + rb * VROW + ((ch ^ swz<NCV, true>(rb)) * 16) + within);
            vf[d] = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    auto compute = [&](int k0, const u32x4 (&kc_)[2][KQ], const bf16x8 (&vf)[DBV]) {

#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            // S^T for 32 keys: two 16-key blocks
            f32x4 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KQ; ++kk)
                    sacc[kb] = mma16<F16>(__builtin_bit_cast(bf16x8, kc_[kb][kk]), qf[cb][kk], sacc[kb]);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = sacc[kb][i];
                    if (p.softcap_on) {
                        const float e = exp2_fast(x * p.c_tanh);
                        x = p.c_cap - 2.f * p.c_cap * __builtin_amdgcn_rcpf(e + 1.f);
                    } else {
                        x *= p.c_score;
                    }
                    if (k0 + kb * 16 + grp * 4 + i > lim[cb]) x = -INFINITY;
                    sacc[kb][i] = x;
                    mx = fmaxf(mx, x);
                }
            }
            mx = quarterwave_max(mx);
            const bool upd = mx > m_run[cb] + kTau;
            if (__builtin_amdgcn_ballot_w64(upd)) {
                const float alpha = upd ? exp2_fast(m_run[cb] - mx) : 1.f;
                m_run[cb] = upd ? mx : m_run[cb];
                l_run[cb] *= alpha;
#pragma unroll
                for (int d = 0; d < DBV; ++d) oacc[cb][d] *= alpha;
            }
            const float nm = (m_run[cb] == -INFINITY) ? 0.f : -m_run[cb];
            // P^T operand: keys (grp*4 + i) of block 0 then of block 1
            uint32_t pk[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                pk[2 * kb] = pack_op2<F16>(exp2_fast(sacc[kb][0] + nm), exp2_fast(sacc[kb][1] + nm));
                pk[2 * kb + 1] = pack_op2<F16>(exp2_fast(sacc[kb][2] + nm), exp2_fast(sacc[kb][3] + nm));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) l_run[cb] = add_op2<F16>(pk[j], l_run[cb]);
            const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
            // O^T += V^T P^T
#pragma unroll
            for (int d = 0; d < DBV; ++d) oacc[cb][d] = mma16<F16>(vf[d], pb, oacc[cb][d]);
        }
    };
    auto prefetch = [&](int k0, u32x4 (&kr)[2][KQ], int st) {
        int bA, bB;
        step_blocks(k0, bA, bB);
        kload(k0, bA, bB, kr);
        vload(k0, bA, bB, st);
    };

    // Two K register buffers alternate (the loop is unrolled by two so no
    // buffer is ever copied while its loads may still be in flight).
    // Each step first waits for its own loads, reads its V^T fragments out of LDS, and only then
    // issues the next step's loads, which run under the step's arithmetic. A transposing LDS read
    // cannot be told apart from the direct-to-LDS copies in flight, so the compiler waits for all
    // of them before one: reading a step's V^T while the next step's copies were in flight made
    // every step wait for those copies before its arithmetic (64 sequences of 1024..8192 keys,
    // 64:8 heads: d = 64 145 -> 123 us, d = 128 248 -> 244 us, d = 192 353 -> 343 us).
    u32x4 kA[2][KQ], kB[2][KQ];
    bf16x8 vf[DBV];
    const int nsteps = (end - start + 31) / 32;
    prefetch(start, kA, 0);
    for (int it = 0; it < nsteps; it += 2) {
        const int k0 = start + it * 32;
        wait_vmem();  // step k0's K fragments and V rows have landed
        vread(0, vf);
        __builtin_amdgcn_sched_barrier(0);
        if (it + 1 < nsteps) prefetch(k0 + 32, kB, 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(k0, kA, vf);
        if (it + 1 >= nsteps) break;
        wait_vmem();
        vread(1, vf);
        __builtin_amdgcn_sched_barrier(0);
        if (it + 2 < nsteps) prefetch(k0 + 64, kA, 0);
        __builtin_amdgcn_sched_barrier(0);
        compute(k0 + 32, kB, vf);
    }

#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const float l_tot = quarterwave_sum(l_run[cb]);
        const int colq = cg0 + cb * 16 + c16;
        if (colq < p.nq) {
            const int si = colq / p.group;
            const int h = g * p.group + colq % p.group;
            const size_t row = ((size_t)b * p.Sq + si) * p.Hq + h;
            const size_t slot = row * p.n_split + split;
            if (grp == 0) {
                p.ws_ml[slot * 2] = m_run[cb];
                p.ws_ml[slot * 2 + 1] = l_tot;
            }
            float* op = p.ws_o + slot * DV;
#pragma unroll
            for (int d = 0; d < DBV; ++d) *(f32x4*)(op + d * 16 + grp * 4) = oacc[cb][d];
        }
    }
}

// Gathered mode: one workgroup per (key split, group of NW*16 heads, token).
// The selected rows of the token are gathered straight from the row cache in
// their native layout (the approach of the "MLA Decode Attention Kernel API
// Reference" page, Background: no pre-gathered copy), 32 rows per step, into
// a ring of NST LDS stages shared by the NW waves (NST-1 steps in flight);
// each wave owns 16 heads (the query columns of its 16x16x32 MFMAs) and the
// whole value width. When the value is a prefix of the key row (VK) the rows
// are loaded once and the value operand is read from the key stage. A key is
// live iff its position is at or before the token's.
//
// Stage layout: 32 rows at a pitch of one row (DK*2 bytes, 128 mod 256), so
// each 1 KB direct load reads contiguous global memory. Row r stores its
// logical 16-byte chunk c at c ^ sw(r) (sw(r) < 8 permutes within aligned
// groups of 8 chunks), and every address is one of a few per-lane bases plus
// an immediate:
//   K operand: a 128-bit read of one chunk by 16 consecutive rows;
//   V^T operand: a transposing read of 4 consecutive rows x 32 bytes.
// The LDS serves a 128-bit read to lanes 0-7 with 32-39 in one cycle (then
// 8-15 with 40-47, ...) and a 64-bit read to 32 consecutive lanes; under that
// grouping (measured with the bank-conflict counter on these exact address
// patterns) sw(r) = r1 | (r1^r2) << 1 | (r2^r3) << 2 makes both reads
// conflict-free. (A plain bit permutation left the K reads 2-way conflicted.)
struct GatherParams {
    const void* __restrict__ q;  // bf16, fp32 or fp16 (q_type)
    const uint16_t* __restrict__ kc;
    const uint16_t* __restrict__ vc;
    float* __restrict__ ws_o;
    float* __restrict__ ws_ml;
    const int32_t* __restrict__ row_index;
    const float* __restrict__ key_pos;
    const int32_t* __restrict__ q_pos;
    // token t's own key row at kc + kcur_off + t * row_stride, value row at vc + vcur_off + ...
    // (element offsets from the cache bases, so every gather address derives from one base pointer)
    long long kcur_off, vcur_off;
    int has_cur;
    int T, Hq, n_sel, n_split, split_len;
    long long row_stride;  // elements
    float c_score, c_tanh, c_cap;
    int causal, softcap_on;
    int q_type;
};

// keys per split the LDS index table holds: a split of up to 1024 selected keys, plus the
// token's own row in the last split, rounded up to whole 32-key steps
constexpr int kGatherMaxSplit = 1024 + 32;

#ifndef ATTN_GPF_K
#define ATTN_GPF_K 4  // K fragments read ahead of their MFMA
#endif
#ifndef ATTN_GPF_V
#define ATTN_GPF_V 4  // V^T fragments read ahead of their MFMA
#endif

// Wait until at most `later` stages of LPS direct loads per wave are still in flight.
template <int LPS>
__device__ __forceinline__ void wait_stages(int later) {
    if (later >= 2)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPS) : "memory");
    else if (later == 1)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS) : "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int DK, int DV, int NW, bool VK, bool F16, bool CAUSAL, bool SOFTCAP>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1)))
void decode_gathered_split_kernel(GatherParams p) {
    constexpr int NT = NW * 64;
    constexpr int KQ = DK / 32;   // QK k-steps of 32 dims
    constexpr int DBV = DV / 16;  // 16-column blocks of O^T
    constexpr int PITCH = DK * 2;             // LDS row pitch (bytes), key and value stages alike
    constexpr int NCH = DK / 8;               // 16-byte chunks per row
    constexpr int SSTAGE = 32 * PITCH;        // one stage of 32 rows
    constexpr int NSEG = SSTAGE / 1024;       // 1 KB direct loads per stage
    constexpr int STAGE = SSTAGE * (VK ? 1 : 2);
    constexpr int NST = VK ? 4 : 2;
    constexpr int LPS = (NSEG / NW) * (VK ? 1 : 2);  // direct loads per wave per stage
    static_assert(DK % 32 == 0 && DV % 64 == 0 && DV <= DK && PITCH % 128 == 0 && PITCH % 256 != 0, "shape");
    static_assert(SSTAGE % 1024 == 0 && NSEG % NW == 0 && NCH % 8 == 0, "stage");
    static_assert(NST * STAGE + 12 * kGatherMaxSplit <= 160 * 1024, "LDS");
    static_assert(NW * 16 * (DV + 4) * 4 <= NST * STAGE, "output staging fits the stages");
    __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];
    __shared__ long long skoff[kGatherMaxSplit];  // element offset of each key row from kc
    __shared__ __attribute__((aligned(16))) float spos[kGatherMaxSplit];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4, c16 = lane & 15;
    const int split = blockIdx.x, hgrp = blockIdx.y, t = blockIdx.z;
    const int start = split * p.split_len;
    const int end = min(p.n_sel, start + p.split_len);
    const int nsel = end - start;
    // the last split also takes the token's own row (n_keys = n_prior + 1), always live
    const int has_cur = (p.has_cur && split == p.n_split - 1) ? 1 : 0;
    const int nk = nsel + has_cur;
    const float qpos = (float)p.q_pos[t];

    // this split's row indices and positions (one per thread per pass)
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
            pos_r[u] = p.key_pos[(size_t)t * p.n_sel + start + i];
        }
    }
    // key rows as element offsets from kc (the token's own row from kcur), and positions
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

    // query fragments (first needed by the first step's QK, so their latency hides
    // under the first stages' copies)
    const int h = hgrp * (NW * 16) + wave * 16 + c16;
    const bool hok = h < p.Hq;
    bf16x8 qf[KQ];
    {
        const size_t qrow = ((size_t)t * p.Hq + (hok ? h : 0)) * DK;
#pragma unroll
        for (int kk = 0; kk < KQ; ++kk) {
            qf[kk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
            if (hok) qf[kk] = load_q8<F16>(p.q, qrow + kk * 32 + grp * 8, p.q_type);
        }
    }

    // row r stores logical chunk c at chunk c ^ sw(r) (within aligned groups of 8)
    auto sw = [](int r) { return ((r >> 1) & 1) | ((((r >> 1) ^ (r >> 2)) & 1) << 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 2); };
    // Rows of step i into stage st: wave w fills 1 KB segments w, w+NW, ... All row offsets
    // of the step are read from LDS before the first copy is issued (a copy writes LDS, so a
    // later table read could not be moved ahead of it).
    constexpr int JW = NSEG / NW;
    auto issue = [&](int i, int st) {
        char* sb = smem + st * STAGE;
        long long ro[JW];
        int kr[JW];
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const int r = ((wave + j * NW) * 1024 + lane * 16) / PITCH;
            kr[j] = min(i * 32 + r, nk - 1);
            ro[j] = skoff[kr[j]];
        }
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const int sg = wave + j * NW;
            const int off = sg * 1024 + lane * 16;
            const int r = off / PITCH;
            const int c = ((off - r * PITCH) >> 4) ^ sw(r);
            load_lds16(p.kc + ro[j] + c * 8, sb + sg * 1024);
            if constexpr (!VK) {
                // value rows use the same layout; chunks past the value width repeat earlier ones
                const long long vo = ro[j] + ((has_cur && kr[j] == nsel) ? p.vcur_off - p.kcur_off : 0);
                load_lds16(p.vc + vo + (c % (DV / 8)) * 8, sb + SSTAGE + sg * 1024);
            }
        }
    };

    // per-lane LDS byte offsets within a stage
    const int sk = sw(c16);  // rows c16 and c16 + 16
    const int kofs0 = c16 * PITCH + ((grp ^ sk) << 4);        // even k-steps (+ kk/2 * 128)
    const int kofs1 = c16 * PITCH + (((4 + grp) ^ sk) << 4);  // odd k-steps
    const int ra = grp * 4 + (c16 >> 2);
    const int sv = sw(ra);
    const int xv = (c16 & 3) >> 1, bv = (c16 & 1) * 8;
    int vofs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vofs[j] = ra * PITCH + (((2 * j + xv) ^ sv) << 4) + bv;

    f32x4 oacc[DBV];
#pragma unroll
    for (int d = 0; d < DBV; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const int nsteps = (nk + 31) / 32;
    for (int j = 0; j < NST - 1 && j < nsteps; ++j) issue(j, j);
#pragma clang loop unroll(disable)
    for (int i = 0; i < nsteps; ++i) {
        wait_stages<LPS>(min(NST - 2, nsteps - 1 - i));
        __syncthreads();
        if (i + NST - 1 < nsteps) issue(i + NST - 1, (i + NST - 1) % NST);
        __builtin_amdgcn_sched_barrier(0);
        const char* kt = smem + (i % NST) * STAGE;
        const char* vt = VK ? kt : kt + SSTAGE;
        const int r0 = i * 32;
        f32x4 kpos[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        if constexpr (CAUSAL) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) kpos[kb] = *(const f32x4*)(spos + r0 + kb * 16 + grp * 4);
        }

        constexpr int NQK = 2 * KQ;
        constexpr int PFK = NQK < ATTN_GPF_K ? NQK : ATTN_GPF_K;
        auto kload = [&](int idx) -> bf16x8 {
            const int kk = idx >> 1, kb = idx & 1;
            const int o = ((kk & 1) ? kofs1 : kofs0) + (kk >> 1) * 128 + kb * 16 * PITCH;
            return *(const bf16x8*)(kt + o);
        };
        f32x4 sacc[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sacc[kb][0] = sacc[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 kring[PFK];
#pragma unroll
        for (int j = 0; j < PFK; ++j) kring[j] = kload(j);
#pragma unroll
        for (int idx = 0; idx < NQK; ++idx) {
            const bf16x8 a = kring[idx % PFK];
            if (idx + PFK < NQK) kring[idx % PFK] = kload(idx + PFK);
            const int kk = idx >> 1, kb = idx & 1;
            sacc[kb][kk & 1] = mma16<F16>(a, qf[kk], sacc[kb][kk & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        f32x4 sc[2];
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sc[kb] = sacc[kb][0] + sacc[kb][1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x = sc[kb][e];
                if constexpr (SOFTCAP) {
                    const float ex = exp2_fast(x * p.c_tanh);
                    x = p.c_cap - 2.f * p.c_cap * __builtin_amdgcn_rcpf(ex + 1.f);
                } else {
                    x *= p.c_score;
                }
                const int kl = r0 + kb * 16 + grp * 4 + e;  // key within the split
                const bool live = kl < nk && (!CAUSAL || kpos[kb][e] <= qpos);
                if (!live) x = -INFINITY;
                sc[kb][e] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = quarterwave_max(mx);
        const bool upd = mx > m_run + kTau;
        if (__builtin_amdgcn_ballot_w64(upd)) {
            const float alpha = upd ? exp2_fast(m_run - mx) : 1.f;
            m_run = upd ? mx : m_run;
            l_run *= alpha;
#pragma unroll
            for (int d = 0; d < DBV; ++d) oacc[d] *= alpha;
        }
        const float nm = (m_run == -INFINITY) ? 0.f : -m_run;
        uint32_t pk[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            pk[2 * kb] = pack_op2<F16>(exp2_fast(sc[kb][0] + nm), exp2_fast(sc[kb][1] + nm));
            pk[2 * kb + 1] = pack_op2<F16>(exp2_fast(sc[kb][2] + nm), exp2_fast(sc[kb][3] + nm));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) l_run = add_op2<F16>(pk[j], l_run);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});

        constexpr int PFV = DBV < ATTN_GPF_V ? DBV : ATTN_GPF_V;
        auto vload = [&](int d) -> bf16x8 {
            const char* pa = vt + vofs[d & 3] + (d >> 2) * 128;
            const bf16x4 va = lds_read_tr16(pa);
            const bf16x4 vb = lds_read_tr16(pa + 16 * PITCH);  // rows + 16
            return __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8 vring[PFV];
#pragma unroll
        for (int j = 0; j < PFV; ++j) vring[j] = vload(j);
#pragma unroll
        for (int d = 0; d < DBV; ++d) {
            const bf16x8 a = vring[d % PFV];
            if (d + PFV < DBV) vring[d % PFV] = vload(d + PFV);
            oacc[d] = mma16<F16>(a, pb, oacc[d]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    const float l_tot = quarterwave_sum(l_run);
    if (hok && grp == 0) {
        const size_t slot = ((size_t)t * p.Hq + h) * p.n_split + split;
        p.ws_ml[slot * 2] = m_run;
        p.ws_ml[slot * 2 + 1] = l_tot;
    }
    // Partial O through LDS (the stages are free once every wave is past its last step), so
    // each store instruction writes 1 KB of contiguous partial row: the wave's 16 heads at a
    // row pitch of DV + 4 floats (conflict-free writes of the O^T fragments).
    constexpr int OP = DV + 4;
    __syncthreads();
    float* ost = (float*)smem + wave * 16 * OP;
#pragma unroll
    for (int d = 0; d < DBV; ++d) *(f32x4*)(ost + c16 * OP + d * 16 + grp * 4) = oacc[d];
    // (a wave's LDS accesses complete in order, so it reads its own writes back directly)
#pragma unroll 4
    for (int k = 0; k < 16 * DV / 256; ++k) {  // 256 floats per instruction
        const int hh = (k * 256) / DV, col = (k * 256) % DV + lane * 4;
        const int head = hgrp * (NW * 16) + wave * 16 + hh;
        if (head < p.Hq) {
            const size_t slot = ((size_t)t * p.Hq + head) * p.n_split + split;
            *(f32x4*)(p.ws_o + slot * DV + col) = *(const f32x4*)(ost + hh * OP + col);
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

// One wavefront per output row (b, query, head). Each lane owns 4 columns (two
// 4-column groups for rows of 512 columns); rows narrower than 256 columns put
// the spare lanes on other splits and add the phases up in LDS. The first 8
// splits of the lane's columns are loaded before the split maxima are read, so
// the row costs one memory latency rather than two; further splits follow 8 at
// a time (indices clamped, values of missing splits zeroed).
template <bool OF32>
__global__ __launch_bounds__(64) void decode_combine_kernel(CombineParams p) {
    constexpr int U = 8;
    constexpr int CL = 2;  // column groups per lane at most (dv <= 512)
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
    const float* ob = p.ws_o + row * p.n_split * p.dv;
    const int ncg = p.dv >> 2;  // 4-column groups
    // lane -> column groups c0 (+64) and split phase ph of G
    const int G = ncg >= 64 ? 1 : 64 / ncg;
    const int ncl = ncg >= 64 ? ncg / 64 : 1;
    const int c0 = ncg >= 64 ? lane : lane % ncg, ph = ncg >= 64 ? 0 : lane / ncg;
    const bool active = ph < G;

    auto load_batch = [&](int s0, f32x4 (&x)[CL][U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * G;
            const int sc = max(min(s, nv - 1), 0);
#pragma unroll
            for (int g = 0; g < CL; ++g) {
                x[g][u] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (active && g < ncl) x[g][u] = *(const f32x4*)(ob + (size_t)sc * p.dv + (c0 + 64 * g) * 4);
            }
        }
    };
    f32x4 x[CL][U];
    load_batch(ph, x);

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

    // sum over the splits s = ph, ph + G, ... (< nv) of e^{m_s - M} O_s
    f32x4 acc[CL];
#pragma unroll
    for (int g = 0; g < CL; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = ph; s0 < nv; s0 += U * G) {
        if (s0 != ph) load_batch(s0, x);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * G;
            const float w = exp2_fast(ml[2 * max(min(s, nv - 1), 0)] - Mu);
#pragma unroll
            for (int g = 0; g < CL; ++g)
                if (s < nv) acc[g] += w * x[g][u];
        }
    }

    auto store = [&](int c, f32x4 a) {
        a *= inv;
        if constexpr (OF32) {
            *(f32x4*)((float*)p.o + row * p.dv + c * 4) = a;
        } else {
            *(u32x2*)((uint16_t*)p.o + row * p.dv + c * 4) =
                u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
        }
    };
    if (ncg >= 64) {
#pragma unroll
        for (int g = 0; g < CL; ++g)
            if (g < ncl) store(c0 + 64 * g, acc[g]);
    } else {  // lanes of phase >= G (when 64 % ncg != 0) only add zeros
        __shared__ f32x4 red[64];
        red[lane] = acc[0];
        __syncthreads();
        if (ph == 0) {
            f32x4 a = acc[0];
            for (int q = 1; q < G; ++q) a += red[q * ncg + c0];
            store(c0, a);
        }
    }
}

// Query columns per workgroup: 16 (one MFMA block) at head dims >= 192, whose registers
// are full, else up to 32; more columns take more workgroups.
inline int paged_cols(int dk, int nq) { return (dk >= 192 || nq <= 16) ? 16 : 32; }

template <int DK, int DV, bool F16>
hipError_t launch_paged_t(const SplitParams& sp, dim3 grid, hipStream_t stream) {
    if (paged_cols(DK, sp.nq) == 16)
        hipLaunchKernelGGL((decode_paged_split_kernel<DK, DV, 1, F16>), grid, dim3(64), 0, stream, sp);
    else if constexpr (DK < 192)
        hipLaunchKernelGGL((decode_paged_split_kernel<DK, DV, 2, F16>), grid, dim3(64), 0, stream, sp);
    return hipGetLastError();
}
template <int DK, int DV>
hipError_t launch_paged(const SplitParams& sp, bool f16, dim3 grid, hipStream_t stream) {
    return f16 ? launch_paged_t<DK, DV, true>(sp, grid, stream) : launch_paged_t<DK, DV, false>(sp, grid, stream);
}

template <int NW, bool VK, bool F16, bool CAUSAL, bool SOFTCAP>
hipError_t launch_gathered_t(const GatherParams& gp, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((decode_gathered_split_kernel<576, 512, NW, VK, F16, CAUSAL, SOFTCAP>), grid, dim3(NW * 64), 0,
                       stream, gp);
    return hipGetLastError();
}
template <int NW, bool VK, bool F16>
hipError_t launch_gathered_f(const GatherParams& gp, bool causal, bool softcap, dim3 grid, hipStream_t stream) {
    if (causal)
        return softcap ? launch_gathered_t<NW, VK, F16, true, true>(gp, grid, stream)
                       : launch_gathered_t<NW, VK, F16, true, false>(gp, grid, stream);
    return softcap ? launch_gathered_t<NW, VK, F16, false, true>(gp, grid, stream)
                   : launch_gathered_t<NW, VK, F16, false, false>(gp, grid, stream);
}
template <int NW>
hipError_t launch_gathered(const GatherParams& gp, bool vk, bool f16, bool causal, bool softcap, dim3 grid,
                           hipStream_t stream) {
    if (vk)
        return f16 ? launch_gathered_f<NW, true, true>(gp, causal, softcap, grid, stream)
                   : launch_gathered_f<NW, true, false>(gp, causal, softcap, grid, stream);
    return f16 ? launch_gathered_f<NW, false, true>(gp, causal, softcap, grid, stream)
               : launch_gathered_f<NW, false, false>(gp, causal, softcap, grid, stream);
}

hipError_t launch_combine(const DecodeArgs& a, const DecodePlan& pl, float* ws_o, float* ws_ml,
                          const int32_t* seq_lens, hipStream_t stream) {
    CombineParams cp;
    cp.ws_o = ws_o;
    cp.ws_ml = ws_ml;
    cp.seq_lens = seq_lens;
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

}  // namespace

bool decode_supported(int dk, int dv, bool gathered) {
    if (gathered) return dk == 576 && dv == 512;
    switch (dk * 1000 + dv) {
        case 16016: case 32032: case 64064: case 96096: case 128128:
        case 192192: case 256256: case 192128:
            return true;
        default:
            return false;
    }
}

DecodePlan decode_plan(int B, int Hq, int Hkv, int Sq, int Sk_max, int dk, int dv) {
    DecodePlan pl;
    if (dk == 576 && dv == 512) {
        // gathered rows: one split per 8 MFMA steps of the 64-head workgroups up to 2048
        // selected keys, longer splits beyond (at most the LDS index table of a split)
        pl.split_len = Sk_max >= 16384 ? 1024 : Sk_max >= 4096 ? 512 : 256;
    } else {
        // paged: one wavefront per (split, KV head, sequence). Aim for about 4096 of them
        // (two rounds of two waves per SIMD) with splits of 256..2048 (4096) keys: long splits
        // when there are many sequences (fewer partial rows to merge), short ones when few
        const long long pairs = (long long)B * Hkv;
        const long long want = (4096 + pairs - 1) / pairs;  // splits per (KV head, sequence)
        long long len = Sk_max > 0 ? (Sk_max + want - 1) / want : 256;
        // The fp32 partials grow with the query columns per KV head, so 32-column groups
        // (paged_cols) take splits of up to 4096 keys (4 tokens x 8 heads, 64 sequences of
        // up to 32K keys: 984 -> 955 us; one token stays at 2048, 8192 was slower for both)
        const int max_sl = paged_cols(dk, Sq * (Hq / Hkv)) == 32 ? 4096 : 2048;
        int sl = 256;
        while (sl < len && sl < max_sl) sl <<= 1;
        pl.split_len = sl;
    }
    pl.n_split = Sk_max > 0 ? (Sk_max + pl.split_len - 1) / pl.split_len : 1;
    pl.n_rows = (int64_t)B * Sq * Hq;
    pl.ws_bytes = (size_t)pl.n_rows * pl.n_split * ((size_t)dv + 2) * sizeof(float);
    pl.ws_bytes = (pl.ws_bytes + 255) & ~(size_t)255;
    return pl;
}

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
    // the device that runs work queued on `stream` (the current device for the null stream)
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (stream != nullptr) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return e;
    }
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        // each GPU holds its own copy of the array at its own address: look it up once per
        // device, with that device current
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
    float* ws_o = (float*)a.workspace;
    float* ws_ml = ws_o + (size_t)pl.n_rows * pl.n_split * a.dv;
    const float kLog2eH = 1.4426950408889634f;

    SplitParams sp;
    sp.q = a.q;
    sp.q_type = a.q_type;
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
    const int cols = paged_cols(a.dk, sp.nq);
    sp.ncg = (sp.nq + cols - 1) / cols;
    int lg = 0;
    while ((1 << lg) < a.block_size) ++lg;
    sp.bs_log2 = lg;
    sp.max_blocks = a.max_blocks;
    sp.n_split = pl.n_split;
    sp.split_len = pl.split_len;
    sp.c_score = a.scale * kLog2eH;
    sp.softcap_on = a.softcap != 0.f;
    sp.c_tanh = sp.softcap_on ? 2.f * a.scale / a.softcap * kLog2eH : 0.f;
    sp.c_cap = a.softcap * kLog2eH;
    sp.causal = a.causal;

    hipError_t e;
    if (a.row_index != nullptr) {
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
        gp.n_sel = a.n_sel;
        gp.n_split = pl.n_split;
        gp.split_len = pl.split_len;
        gp.row_stride = a.row_stride;
        gp.c_score = sp.c_score;
        gp.c_tanh = sp.c_tanh;
        gp.c_cap = sp.c_cap;
        gp.causal = a.causal;
        gp.softcap_on = sp.softcap_on;
        constexpr int NW = 4;
        const dim3 ggrid((unsigned)pl.n_split, (unsigned)((a.Hq + NW * 16 - 1) / (NW * 16)), (unsigned)a.B);
        const bool vk = a.v_cache == a.k_cache;
        e = launch_gathered<NW>(gp, vk, a.kv_f16 != 0, a.causal != 0, sp.softcap_on != 0, ggrid, stream);
        if (e != hipSuccess) return e;
        return launch_combine(a, pl, ws_o, ws_ml, nullptr, stream);
    }
    const dim3 grid((unsigned)(a.Hkv * sp.ncg), (unsigned)a.B, (unsigned)pl.n_split);
    switch (a.dk * 1000 + a.dv) {
        case 16016: e = launch_paged<16, 16>(sp, a.kv_f16 != 0, grid, stream); break;
        case 32032: e = launch_paged<32, 32>(sp, a.kv_f16 != 0, grid, stream); break;
        case 64064: e = launch_paged<64, 64>(sp, a.kv_f16 != 0, grid, stream); break;
        case 96096: e = launch_paged<96, 96>(sp, a.kv_f16 != 0, grid, stream); break;
        case 128128: e = launch_paged<128, 128>(sp, a.kv_f16 != 0, grid, stream); break;
        case 192192: e = launch_paged<192, 192>(sp, a.kv_f16 != 0, grid, stream); break;
        case 256256: e = launch_paged<256, 256>(sp, a.kv_f16 != 0, grid, stream); break;
        case 192128: e = launch_paged<192, 128>(sp, a.kv_f16 != 0, grid, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;

    return launch_combine(a, pl, ws_o, ws_ml, a.seq_lens, stream);
}

}  // namespace attn
