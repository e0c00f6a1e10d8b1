"""Seeded synthetic inputs for the attention path.

This module only draws random numbers and builds index structure (block
tables, row selections, positions). It holds none of the attention arithmetic;
both the HIP path's tests/benchmark and the CPU oracle consume what it returns.
Every tensor of bf16 values is returned as uint16 bit patterns, produced from
fp32 draws by round-to-nearest-even.

Recipe (numpy PCG64, seeded per case): every bf16 tensor is drawn in
4M-element chunks, chunk i of tensor `tag` from the stream
SeedSequence([seed, tag, i]) (q: tag 0, k or the row cache: 1, v: 2); sinks
and all index structure come from one PCG64(seed) stream in the order below.
  * prefill: q, k, v ~ N(0, std^2) (fp32 draw scaled by std, then bf16), then
    sinks ~ N(0, 1) fp32 when requested.
  * paged decode: lengths L_b ~ U{lo..hi} first (they fix the cache size), then
    q, k cache, v cache, then the block table: the N = sum ceil(L_b / bs)
    physical blocks are a random permutation handed out sequence by sequence;
    unused table entries are 0 and never read.
  * gathered decode: row cache ~ N(0,1) of n_rows rows laid out in
    permuted blocks of 64 rows, q, then per token a position q_pos ~
    U{n_sel-1..n_rows-1} and n_sel distinct positions <= q_pos (sorted);
    row_index is the physical row of each position, key_pos its fp32 value.
  * MLA tail: the latent attention output o_lat [T, H, R] ~ N(0, 1) (tag 0),
    out-absorb weights [H, DV, R] ~ N(0, 1/R) (tag 1) and o-projection weights
    [H*DV, N] ~ N(0, 1/(H*DV)) (tag 2), so u and y stay of order 1 (random
    weights of the model's shapes; no trained values).
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "to_bf16_bits",
    "bf16_bits_to_f32",
    "normal_bf16",
    "prefill_case",
    "paged_case",
    "gathered_case",
    "mla_tail_case",
    "CONFIGS",
    "MLA_TAIL",
]


def to_bf16_bits(x):
    """fp32 -> bf16 bit patterns by round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed, tag, shape, std=1.0, chunk=1 << 22, threads=None):
    """N(0, std^2) draws in fp32, rounded to bf16 bits.

    Chunk i of the flattened tensor is drawn from its own PCG64 stream seeded
    by SeedSequence([seed, tag, i]); the result does not depend on how many
    threads draw the chunks.
    """
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)
    starts = list(range(0, n, chunk))

    def work(i):
        s = starts[i]
        e = min(n, s + chunk)
        r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tag), i])))
        x = r.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = to_bf16_bits(x)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if len(starts) <= 1 or threads <= 1:
        for i in range(len(starts)):
            work(i)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(len(starts))))
    return out.reshape(shape)


def normal_typed(seed, tag, shape, dtype, std=1.0):
    """The same N(0, std^2) fp32 draws as normal_bf16, in the element type `dtype`:
    "bf16" (bit patterns, uint16), "f16" (numpy float16, round to nearest even) or
    "f32" (unrounded)."""
    if dtype == "bf16":
        return normal_bf16(seed, tag, shape, std)
    n = int(np.prod(shape)) if len(shape) else 1
    x = np.empty(n, dtype=np.float32)
    for i, s in enumerate(range(0, n, 1 << 22)):
        e = min(n, s + (1 << 22))
        r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tag), i])))
        x[s:e] = r.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x[s:e] *= np.float32(std)
    x = x.reshape(shape)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def prefill_case(seed, B, Sq, Sk, Hq, Hkv, dk, dv, std=1.0, sinks=False):
    """Dense prefill inputs: q [B,Sq,Hq,dk], k [B,Sk,Hkv,dk], v [B,Sk,Hkv,dv] bf16 bits; sinks [Hq] fp32 or None."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = normal_bf16(seed, 0, (B, Sq, Hq, dk), std)
    k = normal_bf16(seed, 1, (B, Sk, Hkv, dk), std)
    v = normal_bf16(seed, 2, (B, Sk, Hkv, dv), std)
    s = rng.standard_normal(Hq, dtype=np.float32) if sinks else None
    return {"q": q, "k": k, "v": v, "sinks": s}


def mask_case(seed, MB, MH, Sq, Sk, width=None, kind="random", p_neg_inf=0.1, std=2.0):
    """Additive fp16 masks [MB, MH, Sq, width] (width >= Sk, default Sk rounded up to a
    multiple of 4; columns >= Sk hold 0).

    kind "random": N(0, std^2) entries, a fraction p_neg_inf of them -inf.
    kind "distance": the position-distance mask used with ALiBi slopes, with query
    i at position Sk - Sq + i: entry -(pos_i - j) for keys j <= pos_i, -inf after
    (causal structure carried by the mask itself).
    """
    width = (Sk + 3) // 4 * 4 if width is None else width
    m = np.zeros((MB, MH, Sq, width), dtype=np.float32)
    if kind == "random":
        rng = np.random.Generator(np.random.PCG64([seed, 7]))
        m[..., :Sk] = rng.standard_normal((MB, MH, Sq, Sk), dtype=np.float32) * std
        m[..., :Sk][rng.random((MB, MH, Sq, Sk)) < p_neg_inf] = -np.inf
    elif kind == "distance":
        pos = np.arange(Sq)[:, None] + (Sk - Sq)
        j = np.arange(Sk)[None, :]
        m[..., :Sk] = np.where(j <= pos, -(pos - j).astype(np.float32), -np.inf)
    else:
        raise ValueError(kind)
    return m.astype(np.float16)


def paged_case(seed, B, Hq, Hkv, dk, dv, len_lo, len_hi, block_size=64, max_blocks=None,
               Sq=1, std=1.0, sinks=False, lens=None):
    """Paged-cache decode inputs.

    Returns q [B,Sq,Hq,dk], k_cache/v_cache [N,Hkv,block_size,d] bf16 bits,
    block_table [B,max_blocks] int32, seq_lens [B] int32, sinks [Hq] or None.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if lens is None:
        lens = rng.integers(len_lo, len_hi, size=B, endpoint=True).astype(np.int32)
    else:
        lens = np.asarray(lens, dtype=np.int32)
    nblk = (lens + block_size - 1) // block_size
    N = int(nblk.sum())
    if max_blocks is None:
        max_blocks = int(max(1, -(-int(len_hi) // block_size)))
    q = normal_bf16(seed, 0, (B, Sq, Hq, dk), std)
    kc = normal_bf16(seed, 1, (max(N, 1), Hkv, block_size, dk), std)
    vc = normal_bf16(seed, 2, (max(N, 1), Hkv, block_size, dv), std)
    s = rng.standard_normal(Hq, dtype=np.float32) if sinks else None
    perm = rng.permutation(N).astype(np.int32)
    table = np.zeros((B, max_blocks), dtype=np.int32)
    pos = 0
    for b in range(B):
        n = int(nblk[b])
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return {"q": q, "k_cache": kc, "v_cache": vc, "block_table": table, "seq_lens": lens,
            "sinks": s, "block_size": block_size}


def gathered_case(seed, T, Hq, dk, dv, n_rows, n_sel, row_dim=None, block_rows=64,
                  std=1.0, sinks=False, future_keys=0):
    """Gathered-row decode inputs (one shared KV head per row).

    kv [n_rows, row_dim] bf16 bits (row_dim defaults to dk; the key is the
    first dk columns, the value the first dv columns); q [T,Hq,dk]; q_pos [T]
    int32; row_index [T,n_sel] int32; key_pos [T,n_sel] fp32.
    future_keys > 0 replaces the last future_keys selections of each token
    with positions q_pos+1 .. q_pos+future_keys (rows that exist but lie after
    the token), so a causal mask on position has something to exclude.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    row_dim = dk if row_dim is None else row_dim
    kv = normal_bf16(seed, 1, (n_rows, row_dim), std)
    q = normal_bf16(seed, 0, (T, Hq, dk), std)
    s = rng.standard_normal(Hq, dtype=np.float32) if sinks else None
    nb = n_rows // block_rows
    block_perm = rng.permutation(nb).astype(np.int64)
    hi = n_rows - 1 - future_keys
    q_pos = rng.integers(n_sel - 1, hi, size=T, endpoint=True).astype(np.int32)
    sel = np.empty((T, n_sel), dtype=np.int64)
    for t in range(T):
        chosen = np.sort(rng.choice(int(q_pos[t]) + 1, size=n_sel, replace=False))
        if future_keys:
            chosen[n_sel - future_keys:] = q_pos[t] + 1 + np.arange(future_keys)
        sel[t] = chosen
    row_index = (block_perm[sel // block_rows] * block_rows + sel % block_rows).astype(np.int32)
    key_pos = sel.astype(np.float32)
    return {"kv": kv, "q": q, "q_pos": q_pos, "row_index": row_index, "key_pos": key_pos,
            "sinks": s}


def mla_tail_case(seed, T, H, R, DV, N):
    """MLA tail inputs: o_lat [T,H,R], w_absorb [H,DV,R], w_o [H*DV,N], all bf16 bits."""
    return {"o_lat": normal_bf16(seed, 0, (T, H, R)),
            "w_absorb": normal_bf16(seed, 1, (H, DV, R), std=R ** -0.5),
            "w_o": normal_bf16(seed, 2, (H * DV, N), std=(H * DV) ** -0.5)}


# The five workloads the path is measured and checked on. Each entry says what
# its inputs are; seeds 1..5.
CONFIGS = {
    "c1_single_head_d16": dict(kind="prefill", seed=1, B=1, Sq=128, Sk=128, Hq=1, Hkv=1, dk=16, dv=16,
                               std=1.0, causal=False, softcap=0.0, sinks=False, scale=0.25, o_dtype="f32"),
    "c2_causal_mha_d128": dict(kind="prefill", seed=2, B=2, Sq=4096, Sk=4096, Hq=32, Hkv=32, dk=128, dv=128,
                               std=1.0, causal=True, softcap=0.0, sinks=False, scale=128 ** -0.5, o_dtype="bf16"),
    "c3a_gqa_d256": dict(kind="prefill", seed=3, B=1, Sq=4096, Sk=4096, Hq=64, Hkv=8, dk=256, dv=256,
                         std=0.5, causal=False, softcap=0.0, sinks=True, scale=1.0 / 16, o_dtype="bf16"),
    "c3b_gqa_d256_causal_softcap": dict(kind="prefill", seed=3, B=1, Sq=4096, Sk=4096, Hq=64, Hkv=8, dk=256,
                                        dv=256, std=0.5, causal=True, softcap=50.0, sinks=True, scale=1.0 / 16,
                                        o_dtype="bf16"),
    "c4_paged_gqa_decode": dict(kind="paged", seed=4, B=64, Hq=64, Hkv=8, dk=128, dv=128, len_lo=1024,
                                len_hi=32768, block_size=64, scale=128 ** -0.5, causal=False, softcap=0.0,
                                sinks=False, o_dtype="bf16"),
    "c5_gathered_mla_decode": dict(kind="gathered", seed=5, T=16, Hq=128, dk=576, dv=512, n_rows=65536,
                                   n_sel=2048, row_dim=576, scale=1.0 / 24, causal=True, softcap=0.0,
                                   sinks=False, o_dtype="bf16"),
}

# The tail that follows the gathered MLA decode: its 16 tokens x 128 heads of
# 512-wide latent output, v_head_dim 128 and hidden width 7168 (DeepSeek-V3's
# published model shape; the page names the model but not the widths), seed 6.
MLA_TAIL = dict(seed=6, T=16, H=128, R=512, DV=128, N=7168)
