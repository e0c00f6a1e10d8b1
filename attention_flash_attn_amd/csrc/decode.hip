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
    constexpr bool LEAN = DK <= 128;        // two waves per SIMD: the lean step below
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
    const int end = start + min(L - start, p.split_len);
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
    // the smallest limit of the wave: a step ending at or before it needs no masking
    int lim_lo = lim[0];
#pragma unroll
    for (int cb = 1; cb < CB; ++cb) lim_lo = min(lim_lo, lim[cb]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lim_lo = min(lim_lo, __shfl_xor(lim_lo, off));
    lim_lo = __builtin_amdgcn_readfirstlane(lim_lo);

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
                    if ((LEAN && DKP == DK) || dk0 < DK)
                        kr[kb][kk] = *(const u32x4*)(base + (size_t)(ro + (uint32_t)(dk0 * 2)));
                    else
                        kr[kb][kk] = u32x4{0, 0, 0, 0};
                }
            } else {
                const uint16_t* r = p.kc + row_off(k0, k0 + kb * 16 + c16, blkA, blkB) * DK;
#pragma unroll
                for (int kk = 0; kk < KQ; ++kk) {
                    const int dk0 = kk * 32 + grp * 8;
                    if ((LEAN && DKP == DK) || dk0 < DK)
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
    // LEAN (two waves per SIMD): softcapped scores are transformed to log2 units before the
    // mask (one uniform branch); otherwise the raw product is masked and maximised, and the
    // positive scale cs joins the exponent's fused multiply-add (cs = 1 for softcapped scores).
    // A step ending at or before lim_lo is visible to every column and skips the mask. The
    // one-wave instances (head dims >= 192) keep the per-score form: the lean one measured
    // 2.5-6% slower there.
    const float cs = p.softcap_on ? 1.f : p.c_score;
    auto compute = [&](int k0, const u32x4 (&kc_)[2][KQ], const bf16x8 (&vf)[DBV]) {
        const bool full = LEAN && k0 + 31 <= lim_lo;
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
            if constexpr (LEAN) {
                if (p.softcap_on) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float e = exp2_fast(sacc[kb][i] * p.c_tanh);
                            sacc[kb][i] = p.c_cap - 2.f * p.c_cap * __builtin_amdgcn_rcpf(e + 1.f);
                        }
                }
                if (!full) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (k0 + kb * 16 + grp * 4 + i > lim[cb]) sacc[kb][i] = -INFINITY;
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[kb][i]);
                mx = quarterwave_max(mx) * cs;  // -inf stays -inf
            } else {
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
            }
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
                float e[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    e[i] = exp2_fast(LEAN ? fmaf(sacc[kb][i], cs, nm) : sacc[kb][i] + nm);
                pk[2 * kb] = pack_op2<F16>(e[0], e[1]);
                pk[2 * kb + 1] = pack_op2<F16>(e[2], e[3]);
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

struct CombineParams {
    const void* __restrict__ ws_o;  // fp32 O_s (paged) or bf16 O_s / l_s (gathered)
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
        nv = min(p.n_split, L > 0 ? (L - 1) / p.split_len + 1 : 0);  // no overflow at long splits
    }
    const float* ml = p.ws_ml + row * p.n_split * 2;
    const float* ob = (const float*)p.ws_o + row * p.n_split * p.dv;
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

// Combine of the gathered mode's ranges: the partial rows are 512 bf16 columns holding O_s / l_s,
// merged with weights l_s e^{m_s - M}. One wavefront per output row (token, head); lane i owns
// columns 8i .. 8i+7 (one 16-byte load per range). The first 8 ranges and their (max, sum)
// pairs are loaded together; further ranges follow 8 at a time (indices clamped, weights of
// missing ranges zero).
template <bool OF32>
__global__ __launch_bounds__(64) void decode_combine_norm_kernel(CombineParams p) {
    constexpr int DV = 512, U = 8;
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const int lane = threadIdx.x;
    const size_t row = blockIdx.x;
    const int h = (int)(row % p.Hq);
    const int nv = p.n_split;
    // lane u < 8 of a batch loads the (max, sum) pair of range s0 + u with the batch's row loads
    // (one memory latency per row); v_readlane hands the pairs to every lane
    const float* ml = p.ws_ml + row * nv * 2;
    const uint16_t* ob = (const uint16_t*)p.ws_o + row * nv * DV + lane * 8;
    u32x4 x[U];
    f32x2_t mlv;
    auto load_batch = [&](int s0) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            x[u] = __builtin_nontemporal_load((const u32x4*)(ob + (size_t)min(s0 + u, nv - 1) * DV));
        mlv = *(const f32x2_t*)(ml + 2 * min(s0 + (lane & (U - 1)), nv - 1));
    };
    auto pair_m = [&](int u) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mlv[0]), u)); };
    auto pair_l = [&](int u) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mlv[1]), u)); };
    load_batch(0);
    float M = -INFINITY;  // clamped repeats of the last range do not change the maximum
#pragma unroll
    for (int u = 0; u < U; ++u) M = fmaxf(M, pair_m(u));
    if (nv > U) {  // more than one batch: the other maxima first
        float mx = -INFINITY;
        for (int s = U + lane; s < nv; s += 64) mx = fmaxf(mx, ml[2 * s]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        M = fmaxf(M, mx);
    }
    const bool has_sink = p.sinks != nullptr;
    const float sink2 = has_sink ? p.sinks[h] * kLog2e : -INFINITY;
    const float M2 = fmaxf(M, sink2);
    const float Mu = (M2 == -INFINITY) ? 0.f : M2;
    float l = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nv; s0 += U) {
        if (s0 != 0) load_batch(s0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // range s was stored divided by its own sum: weight l_s 2^(m_s - M)
            const float w = (s0 + u < nv) ? pair_l(u) * exp2_fast(pair_m(u) - Mu) : 0.f;
            l += w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += w * bf16lo_to_f32(x[u][e]);
                acc[2 * e + 1] += w * bf16hi_to_f32(x[u][e]);
            }
        }
    }
    if (has_sink) l += exp2_fast(sink2 - Mu);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if constexpr (OF32) {
        float* o = (float*)p.o + row * DV + lane * 8;
        *(f32x4*)o = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
        *(f32x4*)(o + 4) = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
    } else {
        *(u32x4*)((uint16_t*)p.o + row * DV + lane * 8) =
            u32x4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                  pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
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

hipError_t launch_combine(const DecodeArgs& a, const DecodePlan& pl, void* ws_o, float* ws_ml,
                          const int32_t* seq_lens, bool norm, hipStream_t stream) {
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
    const dim3 grid((unsigned)pl.n_rows);
    if (norm) {  // gathered mode: dv is 512
        if (a.dv != 512) return hipErrorInvalidValue;
        if (a.o_f32)
            hipLaunchKernelGGL((decode_combine_norm_kernel<true>), grid, dim3(64), 0, stream, cp);
        else
            hipLaunchKernelGGL((decode_combine_norm_kernel<false>), grid, dim3(64), 0, stream, cp);
    } else {
        if (a.o_f32)
            hipLaunchKernelGGL((decode_combine_kernel<true>), grid, dim3(64), 0, stream, cp);
        else
            hipLaunchKernelGGL((decode_combine_kernel<false>), grid, dim3(64), 0, stream, cp);
    }
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
    const bool gathered = dk == 576 && dv == 512;
    if (gathered) {
        // gathered rows: one workgroup per (token, 64 heads, key range). Aim for about 256
        // workgroups (one per CU) with ranges of 64..1024 keys (the LDS index table of a range)
        const long long units = (long long)B * gathered_head_groups(Hq);
        const long long want = (256 + units - 1) / units;  // ranges per unit
        const long long len = Sk_max > 0 ? (Sk_max + want - 1) / want : 64;
        int sl = 64;
        while (sl < len && sl < 1024) sl <<= 1;
        pl.split_len = sl;
    } else {
        // paged: one wavefront per (split, KV head, column group, sequence).
        const long long nq = (long long)Sq * (Hkv > 0 ? Hq / Hkv : 1);
        const int cols = paged_cols(dk, (int)(nq < (1 << 30) ? nq : (1 << 30)));
        long long sl;
        if (dk <= 128 && Sk_max >= 16384) {
            // Long contexts at two waves per SIMD (2048 wave slots on the chip): a split that
            // finds no free slot starts late, and late starters set the end of the launch, so
            // the splits are made as short as possible while the expected number of non-empty
            // ones still fits in 90% of the slots. The lengths are device data; taking them
            // spread evenly up to Sk_max, n splits of a full-length sequence leave (n + 1) / 2
            // per sequence on average: units * (n + 1) / 2 <= 0.9 * slots. Split lengths are
            // powers of two up to 1024 keys and multiples of 1024 above.
            // Measured at 64 sequences of 1024..32768 keys, 8 KV heads, d = 128 (one column
            // group), split length against time per call:
            //   one token:      2048: 853-857 us, 3072: 838, 4096: 863, 5120: 922, 6144: 814
            //   4 draft tokens: 3072: 925, 4096: 928-938, 5120: 975, 6144: 868-870, 7168: 937,
            //                   8192: 987
            // (this rule picks 6 splits, 6144 keys: 231 of each XCD's 256 slots), and against
            // the rule below at 8 sequences of 16K..32K keys 158 vs 163 us, 16 of 1K..32K 215 vs
            // 222 us. Lengths much shorter than the assumed spread under-fill the slots: 64
            // sequences averaging 13.4K keys of up to 32K took 718 us against 639 with the rule
            // below.
            long long units = (long long)B * Hkv * ((nq + cols - 1) / cols);
            if (units < 1) units = 1;
            const long long slots = 2048;
            long long n = (18 * slots / units - 10) / 10;  // floor(1.8 * slots / units - 1)
            if (n < 1) n = 1;
            const long long len = (Sk_max + n - 1) / n;
            sl = 256;
            while (sl < len && sl < 1024) sl <<= 1;
            if (sl < len) sl = (len + 1023) / 1024 * 1024;
        } else {
            // Shorter contexts, and head dims above 128 (one wave per SIMD): about 4096
            // wavefronts (B * Hkv * splits), splits of 256..2048 keys (4096 with 32-column
            // groups, whose fp32 partials are twice as large). Against the rule above this was
            // faster at 64 sequences of 1K..8K keys: d = 256 436 vs 455 us, d = 192 335 vs 346,
            // d = 64 with 4 draft tokens 139 vs 141, and at 128 sequences of 512..4096 keys
            // (32:8 heads, d = 128) 229 vs 238 us.
            const long long pairs = (long long)B * Hkv;
            const long long want = (4096 + pairs - 1) / (pairs > 0 ? pairs : 1);
            const long long len = Sk_max > 0 ? (Sk_max + want - 1) / want : 256;
            const long long max_sl = cols == 32 ? 4096 : 2048;
            sl = 256;
            while (sl < len && sl < max_sl) sl <<= 1;
        }
        pl.split_len = (int)(sl < 0x7ffffc00LL ? sl : 0x7ffffc00LL);
    }
    pl.n_split = Sk_max > 0 ? (int)(((long long)Sk_max + pl.split_len - 1) / pl.split_len) : 1;
    pl.n_rows = (int64_t)B * Sq * Hq;
    // partial rows (fp32 O_s, or bf16 O_s / l_s for gathered rows), then (max, sum) per row and split
    pl.ws_bytes = (size_t)pl.n_rows * pl.n_split * ((size_t)dv * (gathered ? 2 : 4) + 2 * sizeof(float));
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
        uint16_t* ws_on = (uint16_t*)a.workspace;
        float* ws_mln = (float*)(ws_on + (size_t)pl.n_rows * pl.n_split * a.dv);
        e = launch_gathered_split(a, pl, ws_on, ws_mln, stream);
        if (e != hipSuccess) return e;
        return launch_combine(a, pl, ws_on, ws_mln, nullptr, true, stream);
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

    return launch_combine(a, pl, ws_o, ws_ml, a.seq_lens, false, stream);
}

}  // namespace attn
