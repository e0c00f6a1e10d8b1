"""Plain fp64 CPU oracle for fused scaled-dot-product attention.

TEST INFRASTRUCTURE. Only the tests, the smoke entry point and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP path:
no kernels, headers, helpers or constants. It takes numpy arrays and returns
numpy arrays; inputs given as bf16 bit patterns are widened exactly.

What it computes is the plain definition of the operation, one (batch, head)
score matrix at a time, with no tiling and no online softmax:

    x_j = scale * <q, k_j>                          raw dot product, then scale
    x_j = softcap * tanh(x_j / softcap)             only when softcap != 0
    x_j = x_j + slope_h * mask[i, j]                only with an additive mask
    keys that the mask excludes (causal, position, length, mask = -inf) are dropped
    m   = max over the live x_j and the head's sink logit (when sinks are given)
    Z   = sum_j exp(x_j - m) + exp(sink - m)
    o   = sum_j exp(x_j - m) * v_j / Z              (0 when no key is live)
    lse = m + ln Z                                  (-inf when nothing is live)

Sources (page titles and sections):
  * "ggml-metal: FA tensor path: gate to the (256, 256) shape" (llama.cpp
    compare page), fa.metal tensor kernel: score step (scale applied to the raw
    accumulator, then softcap as cap*tanh, then the additive mask), the online
    softmax it tiles, the final block "sinks, O /= S" (virtual sink key with no
    value contribution; a row whose sum is zero is written as 0), and the GQA
    head map q_head / (Hq / Hkv).
  * "UMMA FMHA - Multi-K-tile + PV GEMM + Full Pipeline" page, "What's working"
    and "Key lessons learned": the matrix product is the unscaled dot product and
    the 1/sqrt(d) scale is applied afterwards.
  * "MLA Decode Attention Kernel API Reference" page, Background and parameter
    list: rows gathered from a paged cache by a per-token row list, with the
    causal mask driven by each selected key's absolute position against the
    token's own position.

Readings where the pages are silent:
  * softcap: x <- softcap * tanh(x / softcap); 0 disables it.
  * causal prefill with Sq != Sk is bottom-right aligned: query i sits at
    absolute position Sk - Sq + i and sees keys j <= Sk - Sq + i.
  * a sink is a raw fp32 logit per query head: not scaled, not softcapped.
  * a row with no live key and no sink gives o = 0 and lse = -inf; with a sink
    but no live key it gives o = 0 (the sink carries no value).
  * ALiBi: the page passes m0, m1 and n_head_log2 to the kernel and takes the
    slope of head h as m0^(h+1) for h < n_head_log2, else m1^(2(h-n_head_log2)+1);
    how the host derives them is off the page. The reading taken is the ALiBi
    schedule that this exponent pattern produces: n_head_log2 the largest power
    of two <= Hq, m0 = 2^(-max_bias / n_head_log2), m1 = 2^(-max_bias / (2 n_head_log2)).
    max_bias = 0 gives slope 1 (the mask is added as is).
"""

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "dequant_blocks",
    "alibi_slopes",
    "attend_rows",
    "prefill",
    "decode_paged",
    "decode_gathered",
    "mla_tail",
]


def bf16_bits_to_f64(bits):
    """Widen bf16 bit patterns (uint16) to float64 exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("expected uint16 bf16 bit patterns, got %s" % b.dtype)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant_blocks(raw, fmt):
    """Values of a block-quantized buffer (uint8 bytes), float64 [n_blocks * 32].

    The "ggml-metal: FA tensor path" page has quantized K/V turned into fp16 by a
    pre-pass before the fp16 kernels run; the block formats are off that page.
    Reading taken (ggml's two plainest block formats, 32 values per block, an
    IEEE fp16 scale d first, blocks packed back to back):
      "q8_0": 34 bytes = d, then 32 int8 q;              value = d * q
      "q4_0": 18 bytes = d, then 16 bytes of nibbles;     value = d * (q - 8),
              byte j holds value j in its low nibble and value j + 16 in its high one.
    """
    raw = np.asarray(raw, dtype=np.uint8)
    size = {"q8_0": 34, "q4_0": 18}[fmt]
    if raw.size % size:
        raise ValueError("buffer is not a whole number of blocks")
    blk = raw.reshape(-1, size)
    d = blk[:, :2].copy().view(np.float16).astype(np.float64)[:, 0]
    if fmt == "q8_0":
        q = blk[:, 2:].view(np.int8).astype(np.float64)
    else:
        nib = blk[:, 2:]
        q = np.concatenate([nib & 0x0F, nib >> 4], axis=1).astype(np.float64) - 8.0
    return (d[:, None] * q).reshape(-1)


def _as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def alibi_slopes(n_heads, max_bias):
    """Per-head ALiBi slope (float64 [n_heads]); the "ggml-metal: FA tensor path"
    page, fa.metal tensor kernel: base m0 for the first n_head_log2 heads with
    exponent h + 1, base m1 for the rest with exponent 2 (h - n_head_log2) + 1."""
    if max_bias == 0.0:
        return np.ones(n_heads)
    n_log2 = 1
    while n_log2 * 2 <= n_heads:
        n_log2 *= 2
    m0 = 2.0 ** (-max_bias / n_log2)
    m1 = 2.0 ** (-max_bias / 2.0 / n_log2)
    h = np.arange(n_heads)
    return np.where(h < n_log2, m0 ** (h + 1), m1 ** (2 * (h - n_log2) + 1))


def attend_rows(qrows, keys, values, scale, softcap=0.0, sink=None, live=None, bias=None):
    """Attention of a block of query rows against one key/value set.

    qrows [R, dk], keys [N, dk], values [N, dv]; live [R, N] boolean (True =
    key visible to that row) or None for all visible; bias [R, N] an additive
    term (already multiplied by the head's slope; -inf drops the key) or None;
    sink is a scalar logit or None. Returns (o [R, dv], lse [R]) in float64.

    Follows the tensor kernel on the "ggml-metal: FA tensor path" page: raw
    product, scale, softcap, additive mask, softmax with the sink as an extra
    term of the normaliser, division by the sum with the empty-row rule.
    """
    qrows = np.asarray(qrows, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    R, N = qrows.shape[0], keys.shape[0]
    dv = values.shape[1]

    x = (qrows @ keys.T) * scale                    # raw dot product, then scale
    if softcap != 0.0:
        x = softcap * np.tanh(x / softcap)
    if live is None:
        live = np.ones((R, N), dtype=bool)
    if bias is not None:
        bias = np.asarray(bias, dtype=np.float64)
        live = live & (bias > -np.inf)              # a -inf mask entry drops the key
        x = x + np.where(live, bias, 0.0)           # added after the softcap
    x = np.where(live, x, -np.inf)                  # excluded keys drop out

    m = x.max(axis=1) if N > 0 else np.full(R, -np.inf)
    if sink is not None:
        m = np.maximum(m, float(sink))
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(x - m_safe[:, None])                 # exp(-inf) = 0 for masked keys
    Z = e.sum(axis=1)
    if sink is not None:
        Z = Z + np.exp(float(sink) - m_safe)
    num = e @ values
    o = np.zeros((R, dv), dtype=np.float64)
    has_key = live.any(axis=1)
    ok = has_key & (Z > 0)
    o[ok] = num[ok] / Z[ok, None]
    with np.errstate(divide="ignore"):
        lse = np.where(Z > 0, m_safe + np.log(np.where(Z > 0, Z, 1.0)), -np.inf)
    return o, lse


def _causal_live(q_positions, Nk):
    """live[i, j] = key j at or before the query's absolute position."""
    j = np.arange(Nk)
    return j[None, :] <= np.asarray(q_positions)[:, None]


def prefill(q, k, v, scale, causal=False, softcap=0.0, sinks=None,
            rows=None, heads=None, batches=None, mask=None, max_bias=0.0):
    """Dense prefill attention.

    q [B, Sq, Hq, dk], k [B, Sk, Hkv, dk], v [B, Sk, Hkv, dv] (uint16 bf16 bits
    or floats); sinks [Hq] or None. Query head h reads KV head h // (Hq // Hkv)
    (contiguous groups). Causal is bottom-right aligned.
    mask [MB, MH, Sq, >= Sk] (float16 or float; extra columns ignored) is added
    to the scores of batch b, head h from mask[b % MB, h % MH] (the broadcast of
    the page's kernel), times the head's ALiBi slope for max_bias.

    rows / heads / batches optionally restrict the work to a subset (for
    sampled checks at large sizes); the returned arrays then hold only those
    entries, o [nb, nrows, nh, dv] and lse [nb, nh, nrows].
    Returns (o, lse) in float64.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Sq, Hq, dk = q.shape
    _, Sk, Hkv, dv = v.shape
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    heads = range(Hq) if heads is None else list(heads)
    batches = range(B) if batches is None else list(batches)
    o = np.zeros((len(batches), len(rows), len(heads), dv))
    lse = np.zeros((len(batches), len(heads), len(rows)))
    live = _causal_live(rows + (Sk - Sq), Sk) if causal else None
    if mask is not None:
        mask = np.asarray(mask)
        slopes = alibi_slopes(Hq, max_bias)
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            g = h // group
            sink = None if sinks is None else float(np.asarray(sinks, dtype=np.float64)[h])
            bias = None
            if mask is not None:
                mrows = mask[b % mask.shape[0], h % mask.shape[1]][rows][:, :Sk].astype(np.float64)
                bias = slopes[h] * mrows
            ob, lb = attend_rows(q[b, rows, h, :], k[b, :, g, :], v[b, :, g, :],
                                 scale, softcap, sink, live, bias)
            o[bi, :, hi, :] = ob
            lse[bi, hi, :] = lb
    return o, lse


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale, causal=False,
                 softcap=0.0, sinks=None, batches=None):
    """Decode over a paged KV cache.

    q [B, Sq, Hq, dk]; caches [n_blocks, Hkv, block_size, d]; block_table
    [B, max_blocks] int32; seq_lens [B]. Logical key j of sequence b lives at
    cache[block_table[b, j // block_size], g, j % block_size]. Query i of
    sequence b sits at position L_b - Sq + i (bottom-right) when causal.
    Returns (o [nb, Sq, Hq, dv], lse [nb, Hq, Sq]) in float64.
    """
    q = _as_f64(q)
    kc = np.asarray(k_cache)
    vc = np.asarray(v_cache)
    B, Sq, Hq, dk = q.shape
    Hkv, bs = kc.shape[1], kc.shape[2]
    dv = vc.shape[3]
    group = Hq // Hkv
    block_table = np.asarray(block_table)
    seq_lens = np.asarray(seq_lens)
    batches = range(B) if batches is None else list(batches)
    o = np.zeros((len(batches), Sq, Hq, dv))
    lse = np.zeros((len(batches), Hq, Sq))
    for bi, b in enumerate(batches):
        L = int(seq_lens[b])
        j = np.arange(L)
        phys = block_table[b, j // bs]
        slot = j % bs
        live = _causal_live(np.arange(Sq) + (L - Sq), L) if causal else None
        for g in range(Hkv):
            K = _as_f64(kc[phys, g, slot, :])
            V = _as_f64(vc[phys, g, slot, :])
            for h in range(g * group, (g + 1) * group):
                sink = None if sinks is None else float(np.asarray(sinks, dtype=np.float64)[h])
                ob, lb = attend_rows(q[b, :, h, :], K, V, scale, softcap, sink, live)
                o[bi, :, h, :] = ob
                lse[bi, h, :] = lb
    return o, lse


def decode_gathered(q, k_rows, v_rows, row_index, key_pos, q_pos, scale,
                    causal=True, softcap=0.0, sinks=None, tokens=None, k_cur=None, v_cur=None):
    """Decode over rows gathered from a row cache (one shared KV head).

    q [T, Hq, dk]; k_rows [R, dk] and v_rows [R, dv] are the key and value
    fields of the cache rows; row_index [T, n_sel] selects the rows each token
    attends to; key_pos [T, n_sel] (float) is each selected key's absolute
    position and q_pos [T] the token's own. When causal, a key is live iff
    key_pos <= q_pos. k_cur [T, dk] / v_cur [T, dv] (both or neither) append the
    token's own row as one more key at position q_pos, always live: the
    "MLA Decode Attention Kernel API Reference" page, Dimensions (n_keys =
    n_prior + 1, the selected prior plus the current token) and kv_row_cur.
    Returns (o [nt, Hq, dv], lse [nt, Hq]) in float64.
    """
    q = _as_f64(q)
    k_rows = np.asarray(k_rows)
    v_rows = np.asarray(v_rows)
    T, Hq, dk = q.shape
    dv = v_rows.shape[1]
    row_index = np.asarray(row_index)
    key_pos = np.asarray(key_pos, dtype=np.float64)
    q_pos = np.asarray(q_pos)
    tokens = range(T) if tokens is None else list(tokens)
    o = np.zeros((len(tokens), Hq, dv))
    lse = np.zeros((len(tokens), Hq))
    for ti, t in enumerate(tokens):
        r = row_index[t]
        K = _as_f64(k_rows[r])
        V = _as_f64(v_rows[r])
        live_row = (key_pos[t] <= float(q_pos[t])) if causal else np.ones(len(r), dtype=bool)
        if k_cur is not None:
            K = np.concatenate([K, _as_f64(np.asarray(k_cur)[t])[None, :]])
            V = np.concatenate([V, _as_f64(np.asarray(v_cur)[t])[None, :]])
            live_row = np.concatenate([live_row, [True]])
        for h in range(Hq):
            sink = None if sinks is None else float(np.asarray(sinks, dtype=np.float64)[h])
            ob, lb = attend_rows(q[t, h][None, :], K, V, scale, softcap, sink, live_row[None, :])
            o[ti, h, :] = ob[0]
            lse[ti, h] = lb[0]
    return o, lse


def mla_tail(o_lat, w_absorb, w_o):
    """The two projections after MLA decode attention, per token.

    "MLA Decode Attention Kernel API Reference" page, Background and the
    out_absorb_w / o_proj_w parameters: the attention output of head h lives in
    the cache's latent space (width R = kv_lora_rank); the head's slice of the
    out-absorb weight [DV, R] maps it to v_head_dim values, and the o-projection
    [H * DV, N] maps the heads' values, head after head, to the hidden width:

        u[t, h, v] = sum_c w_absorb[h, v, c] * o_lat[t, h, c]
        y[t, n]    = sum_h sum_v u[t, h, v] * w_o[h * DV + v, n]

    o_lat [T, H, R], w_absorb [H, DV, R], w_o [H * DV, N] (bf16 bit patterns or
    floats). Returns (y [T, N], u [T, H, DV]) in float64, nothing rounded.
    """
    o = _as_f64(o_lat)
    wa = _as_f64(w_absorb)
    wo = _as_f64(w_o)
    T, H, R = o.shape
    DV = wa.shape[1]
    if wa.shape != (H, DV, R) or wo.shape[0] != H * DV:
        raise ValueError("shape mismatch: o_lat %s, w_absorb %s, w_o %s" % (o.shape, wa.shape, wo.shape))
    u = np.empty((T, H, DV))
    for h in range(H):
        u[:, h, :] = o[:, h, :] @ wa[h].T
    y = u.reshape(T, H * DV) @ wo
    return y, u
