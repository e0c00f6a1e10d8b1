"""Pins for the CPU oracle: facts fixed by the pages and by mathematics.

Each pin takes an oracle module (the real one, or a copy with a planted
mistake) and raises AssertionError when the oracle disagrees with the fact.
None of them retypes the oracle's formula: they use the pages' worked example,
a scalar 40-digit brute force written separately, torch's own SDPA routine,
closed forms and invariants.
"""

import json
import math
import os

import numpy as np

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, "%s: max abs err %.3e > %.1e" % (what, err, tol)


# ---------------------------------------------------------------- pages' numbers
def pin_worked_example(orc):
    """All-ones Q, K at head dim 16: every scaled score is 4.0 (the page's value),
    so the softmax is uniform: lse = 4.0 + ln(Sk) and o = mean of the V rows."""
    with open(os.path.join(GOLDEN, "worked_example_hd16_all_ones.json")) as f:
        g = json.load(f)
    d, n = g["head_dim"], g["key_count"]
    q = np.ones((1, n, 1, d))
    k = np.ones((1, n, 1, d))
    v = _rand(_rng(11), 1, n, 1, d)
    o, lse = orc.prefill(q, k, v, g["scale"])
    _close(lse, np.full((1, 1, n), g["scaled_score"] + math.log(n)), 1e-12, "lse of all-ones case")
    _close(o[0, :, 0, :], np.broadcast_to(v[0, :, 0, :].mean(axis=0), (n, d)), 1e-12, "uniform average")


# ---------------------------------------------------------------- brute force
def _brute_compare(orc, B, Sq, Sk, Hq, Hkv, dk, dv, causal, softcap, sinks, seed):
    rng = _rng(seed)
    q = _rand(rng, B, Sq, Hq, dk)
    k = _rand(rng, B, Sk, Hkv, dk)
    v = _rand(rng, B, Sk, Hkv, dv)
    s = _rand(rng, Hq) if sinks else None
    scale = 1.0 / math.sqrt(dk)
    o, lse = orc.prefill(q, k, v, scale, causal=causal, softcap=softcap, sinks=s)
    ob, lb = brute.prefill_decimal(q.tolist(), k.tolist(), v.tolist(), scale, causal, softcap,
                                   None if s is None else s.tolist())
    ob = np.array([[[[float(x) for x in row] for row in hh] for hh in ii] for ii in ob])
    lb = np.array([[[(-math.inf if x is None else float(x)) for x in r] for r in hh] for hh in lb])
    _close(o, ob, 1e-12, "o vs decimal brute force")
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse)), "lse -inf pattern differs from brute force"
    _close(lse[fin], lb[fin], 1e-12, "lse vs decimal brute force")


def pin_brute_plain(orc):
    _brute_compare(orc, 2, 5, 7, 2, 2, 4, 3, False, 0.0, False, 21)


def pin_brute_causal_gqa(orc):
    _brute_compare(orc, 1, 6, 6, 4, 2, 5, 4, True, 0.0, False, 22)


def pin_brute_causal_rect(orc):
    """Sq < Sk: bottom-right alignment (query i at position Sk - Sq + i)."""
    _brute_compare(orc, 1, 3, 8, 2, 1, 4, 2, True, 0.0, False, 23)


def pin_brute_softcap_sinks(orc):
    _brute_compare(orc, 1, 4, 6, 4, 2, 3, 3, True, 0.7, True, 24)


def pin_brute_empty_rows(orc):
    """Sq > Sk with causal: the first rows see no key (o = 0, lse = -inf)."""
    _brute_compare(orc, 1, 6, 3, 1, 1, 3, 2, True, 0.0, False, 25)


# ---------------------------------------------------------------- library routine
def pin_torch_sdpa(orc):
    """Without softcap and sinks the op is torch's scaled_dot_product_attention
    (fp64, CPU, explicit bottom-right boolean mask, GQA by enable_gqa)."""
    import torch
    rng = _rng(31)
    B, Sq, Sk, Hq, Hkv, dk, dv = 2, 9, 13, 6, 2, 16, 8
    q = _rand(rng, B, Sq, Hq, dk)
    k = _rand(rng, B, Sk, Hkv, dk)
    v = _rand(rng, B, Sk, Hkv, dv)
    for causal in (False, True):
        o, _ = orc.prefill(q, k, v, 0.3, causal=causal)
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)
        tk = torch.from_numpy(k).permute(0, 2, 1, 3)
        tv = torch.from_numpy(v).permute(0, 2, 1, 3)
        mask = None
        if causal:
            i = torch.arange(Sq)[:, None]
            j = torch.arange(Sk)[None, :]
            mask = j <= i + (Sk - Sq)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.3,
                                                               enable_gqa=True)
        _close(o, ref.permute(0, 2, 1, 3).numpy(), 1e-12, "vs torch sdpa causal=%s" % causal)


# ---------------------------------------------------------------- invariants / closed forms
def pin_prob_rows(orc):
    """With V = identity (dv = Sk) the output row is the probability row itself:
    non-negative, summing to 1 (to 1 - sigma with a sink), zero on masked keys."""
    rng = _rng(41)
    Sq = Sk = 7
    q = _rand(rng, 1, Sq, 1, 4)
    k = _rand(rng, 1, Sk, 1, 4)
    v = np.eye(Sk).reshape(1, Sk, 1, Sk)
    o, _ = orc.prefill(q, k, v, 0.5, causal=True)
    p = o[0, :, 0, :]
    assert (p >= 0).all()
    _close(p.sum(axis=1), np.ones(Sq), 1e-13, "probability rows sum to 1")
    assert np.all(p[np.triu_indices(Sk, 1)] == 0), "masked keys carry probability"


def pin_constant_v(orc):
    rng = _rng(42)
    q = _rand(rng, 1, 5, 2, 8)
    k = _rand(rng, 1, 9, 1, 8)
    v = np.full((1, 9, 1, 3), 2.5)
    for causal in (False, True):
        o, _ = orc.prefill(q, k, v, 0.4, causal=causal, softcap=1.3)
        _close(o, np.full_like(o, 2.5), 1e-13, "constant V gives constant output")


def pin_key_permutation(orc):
    rng = _rng(43)
    q = _rand(rng, 1, 4, 2, 6)
    k = _rand(rng, 1, 11, 2, 6)
    v = _rand(rng, 1, 11, 2, 5)
    perm = rng.permutation(11)
    o1, l1 = orc.prefill(q, k, v, 0.37, softcap=2.0)
    o2, l2 = orc.prefill(q, k[:, perm], v[:, perm], 0.37, softcap=2.0)
    _close(o1, o2, 1e-13, "key permutation without a mask")
    _close(l1, l2, 1e-13, "lse under key permutation")


def pin_causal_row0(orc):
    rng = _rng(44)
    q = _rand(rng, 2, 6, 3, 4)
    k = _rand(rng, 2, 6, 3, 4)
    v = _rand(rng, 2, 6, 3, 5)
    o, _ = orc.prefill(q, k, v, 0.5, causal=True)
    assert np.array_equal(o[:, 0], v[:, 0]), "causal row 0 must equal V[0] exactly"


def pin_q_zero_mean(orc):
    """q = 0 makes every visible score equal: the output is the mean of the visible V rows."""
    rng = _rng(45)
    Sq, Sk = 3, 7
    q = np.zeros((1, Sq, 1, 4))
    k = _rand(rng, 1, Sk, 1, 4)
    v = _rand(rng, 1, Sk, 1, 3)
    o, _ = orc.prefill(q, k, v, 0.5, causal=True)
    for i in range(Sq):
        n = Sk - Sq + i + 1
        _close(o[0, i, 0], v[0, :n, 0].mean(axis=0), 1e-13, "mean of the first %d rows" % n)


def pin_sq1_full(orc):
    """A single query (the last position) sees every key whether or not causal is set."""
    rng = _rng(46)
    q = _rand(rng, 1, 1, 2, 8)
    k = _rand(rng, 1, 10, 2, 8)
    v = _rand(rng, 1, 10, 2, 4)
    o1, _ = orc.prefill(q, k, v, 0.35, causal=True)
    o2, _ = orc.prefill(q, k, v, 0.35, causal=False)
    _close(o1, o2, 0.0, "Sq = 1 causal equals full")


def pin_softcap_limit_and_bound(orc):
    rng = _rng(47)
    q = _rand(rng, 1, 6, 1, 8, std=3.0)
    k = _rand(rng, 1, 6, 1, 8, std=3.0)
    v = np.eye(6).reshape(1, 6, 1, 6)
    o0, _ = orc.prefill(q, k, v, 0.5)
    o1, _ = orc.prefill(q, k, v, 0.5, softcap=1e30)
    _close(o0, o1, 1e-12, "softcap -> infinity equals no softcap")
    cap = 0.8
    o2, _ = orc.prefill(q, k, v, 0.5, softcap=cap)
    logp = np.log(o2[0, :, 0, :])
    spread = logp.max(axis=1) - logp.min(axis=1)
    assert (spread < 2 * cap + 1e-12).all(), "capped scores must lie in (-cap, cap)"
    # odd symmetry: scores for -q are the negatives, so log p(q) + log p(-q) is constant per row
    o3, _ = orc.prefill(-q, k, v, 0.5, softcap=cap)
    tot = logp + np.log(o3[0, :, 0, :])
    _close(tot - tot.mean(axis=1, keepdims=True), np.zeros_like(tot), 1e-12, "softcap odd symmetry")


def pin_sinks_virtual_key(orc):
    """A sink equals one extra key whose scaled score is the sink logit and whose value is 0."""
    rng = _rng(48)
    B, Sq, Sk, H, d, dv = 1, 5, 6, 2, 4, 3
    scale = 0.6
    q = _rand(rng, B, Sq, H, d)
    k = _rand(rng, B, Sk, H, d)
    v = _rand(rng, B, Sk, H, dv)
    s = _rand(rng, H) * 2
    for causal in (False, True):
        o, lse = orc.prefill(q, k, v, scale, causal=causal, sinks=s)
        for h in range(H):
            qa = np.concatenate([q[:, :, h:h + 1], np.full((B, Sq, 1, 1), 1.0 / scale)], axis=3)
            ka = np.concatenate([k[:, :, h:h + 1], np.zeros((B, Sk, 1, 1))], axis=3)
            sink_key = np.zeros((B, 1, 1, d + 1))
            sink_key[..., d] = s[h]
            ka = np.concatenate([sink_key, ka], axis=1)         # position 0: visible to all
            va = np.concatenate([np.zeros((B, 1, 1, dv)), v[:, :, h:h + 1]], axis=1)
            oa, la = orc.prefill(qa, ka, va, scale, causal=causal)
            _close(o[:, :, h:h + 1], oa, 1e-12, "sink as a virtual key (o)")
            _close(lse[:, h:h + 1], la, 1e-12, "sink as a virtual key (lse)")


def pin_sinks_closed_form(orc):
    """Constant V = c with a sink: o = c * (1 - sigma), sigma = e^sink / (e^sink + sum e^x);
    a sink of -inf-like size changes nothing."""
    rng = _rng(49)
    q = _rand(rng, 1, 3, 1, 4)
    k = _rand(rng, 1, 5, 1, 4)
    v = np.full((1, 5, 1, 2), -1.75)
    sink = np.array([0.9])
    o, lse = orc.prefill(q, k, v, 0.5, sinks=sink)
    o0, lse0 = orc.prefill(q, k, v, 0.5)
    x = 0.5 * np.einsum("id,jd->ij", q[0, :, 0], k[0, :, 0])
    sig = np.exp(sink[0]) / (np.exp(sink[0]) + np.exp(x).sum(axis=1))
    _close(o[0, :, 0, 0], -1.75 * (1 - sig), 1e-13, "sink closed form")
    o2, _ = orc.prefill(q, k, v, 0.5, sinks=np.array([-1e300]))
    _close(o2, o0, 0.0, "sink at -inf equals no sink")


def pin_gqa_repeat(orc):
    rng = _rng(50)
    q = _rand(rng, 1, 5, 8, 4)
    k = _rand(rng, 1, 7, 2, 4)
    v = _rand(rng, 1, 7, 2, 3)
    o1, _ = orc.prefill(q, k, v, 0.5, causal=True)
    o2, _ = orc.prefill(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), 0.5, causal=True)
    _close(o1, o2, 0.0, "GQA equals MHA with repeated KV heads")


def pin_split_merge(orc):
    """Attention over a union of key sets is the lse-weighted merge of the parts."""
    rng = _rng(51)
    q = _rand(rng, 1, 4, 1, 6)
    k = _rand(rng, 1, 12, 1, 6)
    v = _rand(rng, 1, 12, 1, 5)
    o, lse = orc.prefill(q, k, v, 0.45)
    parts = [(0, 5), (5, 6), (6, 12)]
    os_, ls_ = [], []
    for a, b in parts:
        oo, ll = orc.prefill(q, k[:, a:b], v[:, a:b], 0.45)
        os_.append(oo[0, :, 0])
        ls_.append(ll[0, 0])
    L = np.stack(ls_)
    M = L.max(axis=0)
    tot = np.log(np.exp(L - M).sum(axis=0)) + M
    merged = sum(np.exp(ls_[i] - tot)[:, None] * os_[i] for i in range(len(parts)))
    _close(lse[0, 0], tot, 1e-12, "merged lse")
    _close(o[0, :, 0], merged, 1e-12, "merged output")


# ---------------------------------------------------------------- decode modes
def pin_paged(orc):
    """Paged decode equals dense attention over the sequence's first L keys, and the
    physical placement of blocks does not matter."""
    rng = _rng(52)
    B, Hq, Hkv, d, bs = 3, 4, 2, 8, 4
    lens = np.array([5, 12, 1])
    nblk = -(-lens // bs)
    N = int(nblk.sum())
    q = _rand(rng, B, 1, Hq, d)
    dense_k = [_rand(rng, int(L), Hkv, d) for L in lens]
    dense_v = [_rand(rng, int(L), Hkv, d) for L in lens]
    for table_kind in ("identity", "random"):
        order = np.arange(N) if table_kind == "identity" else rng.permutation(N)
        kc = np.zeros((N, Hkv, bs, d))
        vc = np.zeros((N, Hkv, bs, d))
        table = np.zeros((B, 4), dtype=np.int32)
        p = 0
        for b, L in enumerate(lens):
            for j in range(int(nblk[b])):
                phys = order[p]
                p += 1
                table[b, j] = phys
                n = min(bs, int(L) - j * bs)
                kc[phys, :, :n] = dense_k[b][j * bs:j * bs + n].transpose(1, 0, 2)
                vc[phys, :, :n] = dense_v[b][j * bs:j * bs + n].transpose(1, 0, 2)
        o, _ = orc.decode_paged(q, kc, vc, table, lens, 0.4, causal=True)
        for b, L in enumerate(lens):
            od, _ = orc.prefill(q[b:b + 1], dense_k[b][None], dense_v[b][None], 0.4)
            _close(o[b], od[0], 1e-13, "paged vs dense (%s table)" % table_kind)


def pin_paged_multi_token_causal(orc):
    """Several query rows per sequence (a speculative draft) with the causal mask: the
    rows are the sequence's last Sq positions, so query i of a sequence of L keys sees
    exactly its first L - Sq + i + 1 keys (none when that is <= 0, giving o = 0). Each
    row is checked against torch's scaled_dot_product_attention in fp64 over the
    truncated, contiguous key set; the cache is paged through a random block table."""
    import torch
    rng = _rng(54)
    B, Sq, Hq, Hkv, d, bs = 3, 4, 4, 2, 8, 4
    lens = np.array([9, 4, 2])                  # the last sequence has fewer keys than queries
    nblk = -(-lens // bs)
    N = int(nblk.sum())
    q = _rand(rng, B, Sq, Hq, d)
    dense_k = [_rand(rng, int(L), Hkv, d) for L in lens]
    dense_v = [_rand(rng, int(L), Hkv, d) for L in lens]
    order = rng.permutation(N)
    kc = _rand(rng, N, Hkv, bs, d)              # slots past a sequence's end hold noise
    vc = _rand(rng, N, Hkv, bs, d)
    table = np.zeros((B, 3), dtype=np.int32)
    p = 0
    for b, L in enumerate(lens):
        for j in range(int(nblk[b])):
            phys = order[p]
            p += 1
            table[b, j] = phys
            n = min(bs, int(L) - j * bs)
            kc[phys, :, :n] = dense_k[b][j * bs:j * bs + n].transpose(1, 0, 2)
            vc[phys, :, :n] = dense_v[b][j * bs:j * bs + n].transpose(1, 0, 2)
    o, lse = orc.decode_paged(q, kc, vc, table, lens, 0.35, causal=True)
    for b, L in enumerate(lens):
        for i in range(Sq):
            n_vis = int(L) - Sq + i + 1
            for h in range(Hq):
                g = h // (Hq // Hkv)
                if n_vis <= 0:
                    _close(o[b, i, h], np.zeros(d), 0.0, "draft row with no visible key")
                    assert lse[b, h, i] == -np.inf, "lse of a draft row with no visible key"
                    continue
                qt = torch.from_numpy(q[b, i, h][None, None, None, :])
                kt = torch.from_numpy(np.ascontiguousarray(dense_k[b][:n_vis, g])[None, None])
                vt = torch.from_numpy(np.ascontiguousarray(dense_v[b][:n_vis, g])[None, None])
                ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.35)
                _close(o[b, i, h], ref[0, 0, 0].numpy(), 1e-13,
                       "draft row %d of sequence %d (%d visible keys)" % (i, b, n_vis))


def pin_bf16_bit_patterns(orc):
    """Inputs given as bf16 bit patterns (uint16) are widened exactly: hand-worked
    patterns (bf16 is sign, 8 exponent bits with bias 127, 7 fraction bits; the
    all-zero exponent holds subnormals fraction/128 * 2^-126), torch's own
    bfloat16 -> float64 conversion on random bit patterns, and the attention entry
    points giving the same result on bit patterns as on the widened values."""
    import torch
    table = {
        0x3F80: 1.0, 0xC040: -3.0, 0x3E80: 0.25, 0xBF00: -0.5, 0x4049: 3.140625,
        0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133, 0x007F: 127 * 2.0 ** -133, 0x8001: -(2.0 ** -133),
        0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x7F80: np.inf, 0xFF80: -np.inf,
    }
    bits = np.array(list(table), dtype=np.uint16)
    got = orc.bf16_bits_to_f64(bits)
    assert got.dtype == np.float64
    for b, want in zip(bits, got):
        assert want == table[int(b)], "bf16 0x%04X widened to %r, expected %r" % (b, want, table[int(b)])
    z = orc.bf16_bits_to_f64(np.array([0x0000, 0x8000], dtype=np.uint16))
    assert z[0] == 0.0 and z[1] == 0.0 and not np.signbit(z[0]) and np.signbit(z[1]), "signed zeros"
    rb = _rng(81).integers(0, 1 << 16, 4096).astype(np.uint16)
    rb = rb[(rb & 0x7F80) != 0x7F80]            # finite patterns (no inf / NaN)
    ref = torch.from_numpy(rb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.bf16_bits_to_f64(rb), ref), "widening differs from torch's bfloat16 conversion"

    def bits_and_values(shape, seed):
        x = torch.from_numpy(_rand(_rng(seed), *shape)).to(torch.bfloat16)
        return x.view(torch.int16).numpy().view(np.uint16), x.to(torch.float64).numpy()
    qb, qf = bits_and_values((1, 5, 2, 8), 82)
    kb, kf = bits_and_values((1, 6, 1, 8), 83)
    vb, vf = bits_and_values((1, 6, 1, 8), 84)
    o1, l1 = orc.prefill(qb, kb, vb, 0.3, causal=True)
    o2, l2 = orc.prefill(qf, kf, vf, 0.3, causal=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "prefill on bit patterns vs values"
    kcb, kcf = bits_and_values((3, 1, 4, 8), 85)
    vcb, vcf = bits_and_values((3, 1, 4, 8), 86)
    tab = np.array([[2, 0, 1]], dtype=np.int32)
    o1, _ = orc.decode_paged(qb[:, :1], kcb, vcb, tab, np.array([10]), 0.3)
    o2, _ = orc.decode_paged(qf[:, :1], kcf, vcf, tab, np.array([10]), 0.3)
    assert np.array_equal(o1, o2), "paged decode on bit patterns vs values"
    rowb, rowf = bits_and_values((7, 8), 87)
    ri = np.array([[4, 0, 6]], dtype=np.int32)
    o1, _ = orc.decode_gathered(qb[0, :1], rowb, rowb[:, :5], ri, np.array([[1.0, 2.0, 3.0]]), np.array([2]), 0.3)
    o2, _ = orc.decode_gathered(qf[0, :1], rowf, rowf[:, :5], ri, np.array([[1.0, 2.0, 3.0]]), np.array([2]), 0.3)
    assert np.array_equal(o1, o2), "gathered decode on bit patterns vs values"


def pin_gathered(orc):
    """Gathered decode equals dense attention over the selected rows that lie at or
    before the token (a key exactly at the token's position counts), ignores the
    order of the selection, and a future position acts as a deletion."""
    rng = _rng(53)
    R, T, H, dk, dv = 40, 3, 4, 8, 6
    kv = _rand(rng, R, dk)
    q = _rand(rng, T, H, dk)
    q_pos = np.array([20, 9, 33])
    sel_pos = [np.array([0, 3, 20, 7, 25]), np.array([9, 1, 2, 5, 30]), np.array([33, 32, 31, 0, 4])]
    row_of_pos = rng.permutation(R)
    row_index = np.stack([row_of_pos[p] for p in sel_pos]).astype(np.int32)
    key_pos = np.stack(sel_pos).astype(np.float32)
    o, _ = orc.decode_gathered(q, kv, kv[:, :dv], row_index, key_pos, q_pos, 0.3, causal=True)
    for t in range(T):
        keep = sel_pos[t] <= q_pos[t]
        rows = row_of_pos[sel_pos[t][keep]]
        od, _ = orc.prefill(q[t][None, None], kv[rows][None, :, None, :], kv[rows][None, :, None, :dv], 0.3)
        _close(o[t], od[0, 0], 1e-13, "gathered vs dense over live rows")
    perm = rng.permutation(5)
    o2, _ = orc.decode_gathered(q, kv, kv[:, :dv], row_index[:, perm], key_pos[:, perm], q_pos, 0.3)
    _close(o, o2, 1e-13, "selection order")


def pin_gathered_current_row(orc):
    """The current token's row appended as key n_prior (always live) equals the same row
    stored in the cache and selected with position q_pos; and when every prior key lies
    after the token, the current row is the only live key, so o is its value exactly."""
    rng = _rng(71)
    T, Hq, d, R, n_sel = 3, 4, 8, 40, 6
    rows = _rand(rng, R, d)
    q = _rand(rng, T, Hq, d)
    cur = _rand(rng, T, d)
    q_pos = np.array([20, 33, 9])
    sel = np.stack([rng.choice(R, n_sel, replace=False) for _ in range(T)])
    kpos = np.stack([rng.choice(int(q_pos[t]), n_sel, replace=False) for t in range(T)]).astype(np.float64)
    o1, l1 = orc.decode_gathered(q, rows, rows[:, :5], sel, kpos, q_pos, 0.3, k_cur=cur, v_cur=cur[:, :5])
    rows2 = np.concatenate([rows, cur])                       # the current rows stored at R .. R+T-1
    sel2 = np.concatenate([sel, (R + np.arange(T))[:, None]], axis=1)
    kpos2 = np.concatenate([kpos, q_pos[:, None].astype(np.float64)], axis=1)
    o2, l2 = orc.decode_gathered(q, rows2, rows2[:, :5], sel2, kpos2, q_pos, 0.3)
    _close(o1, o2, 1e-13, "appended current row vs stored and selected")
    _close(l1, l2, 1e-13, "lse with the current row")
    future = q_pos[:, None] + 1.0 + np.arange(n_sel)[None, :]
    o3, _ = orc.decode_gathered(q, rows, rows[:, :5], sel, future, q_pos, 0.3, k_cur=cur, v_cur=cur[:, :5])
    _close(o3, np.broadcast_to(cur[:, None, :5], o3.shape), 1e-15, "only the current row is live")


def _block(d, payload):
    return np.concatenate([np.frombuffer(np.float16(d).tobytes(), dtype=np.uint8),
                           np.asarray(payload, dtype=np.uint8)])


def pin_dequant_q8_0(orc):
    """Hand-built q8_0 blocks: scale 0.5 with q = -16..15, then scale -2 with q = 127, -128, 0, ..."""
    q1 = np.arange(-16, 16, dtype=np.int8)
    q2 = np.zeros(32, dtype=np.int8)
    q2[0], q2[1], q2[31] = 127, -128, 3
    raw = np.concatenate([_block(0.5, q1.view(np.uint8)), _block(-2.0, q2.view(np.uint8))])
    want = np.concatenate([0.5 * np.arange(-16, 16), np.zeros(32)])
    want[32], want[33], want[63] = -254.0, 256.0, -6.0
    _close(orc.dequant_blocks(raw, "q8_0"), want, 0.0, "q8_0 values")


def pin_dequant_q4_0(orc):
    """A q4_0 block with scale 0.25: byte j = (hi << 4) | lo gives values j (lo) and j + 16 (hi)."""
    lo = np.arange(16, dtype=np.uint8)            # values 0..15   -> q - 8 = -8..7
    hi = (15 - np.arange(16)).astype(np.uint8)    # values 16..31  -> 7..-8
    raw = _block(0.25, (hi << 4) | lo)
    want = 0.25 * np.concatenate([np.arange(16) - 8.0, 7.0 - np.arange(16)])
    _close(orc.dequant_blocks(raw, "q4_0"), want, 0.0, "q4_0 values")


# ---------------------------------------------------------------- additive mask, ALiBi
def pin_alibi_slopes_published(orc):
    """The ALiBi slope schedule (Press, Smith and Lewis, "Train Short, Test Long"):
    n heads (a power of two) get 2^(-8/n), 2^(-16/n), ..., 2^(-8) for a maximum bias
    of 8; other head counts take the slopes of the nearest smaller power of two,
    then every other slope of twice that count. Written out by hand below."""
    _close(orc.alibi_slopes(8, 8.0), [2.0 ** -e for e in range(1, 9)], 1e-15, "8-head slopes")
    table12 = [2.0 ** -e for e in range(1, 9)] + [2.0 ** -0.5, 2.0 ** -1.5, 2.0 ** -2.5, 2.0 ** -3.5]
    _close(orc.alibi_slopes(12, 8.0), table12, 1e-15, "12-head slopes")
    _close(orc.alibi_slopes(2, 8.0), [2.0 ** -4, 2.0 ** -8], 1e-15, "2-head slopes")
    _close(orc.alibi_slopes(5, 0.0), np.ones(5), 0.0, "max_bias 0 leaves the mask unscaled")


def _mask(rng, MB, MH, Sq, Sk, p_neg_inf=0.15):
    m = _rand(rng, MB, MH, Sq, Sk, std=2.0)
    m[rng.random(m.shape) < p_neg_inf] = -np.inf
    return m


def _brute_mask_compare(orc, B, Sq, Sk, Hq, Hkv, d, MB, MH, softcap, causal, max_bias, slopes, seed):
    rng = _rng(seed)
    q = _rand(rng, B, Sq, Hq, d)
    k = _rand(rng, B, Sk, Hkv, d)
    v = _rand(rng, B, Sk, Hkv, d)
    mask = _mask(rng, MB, MH, Sq, Sk)
    scale = 1.0 / math.sqrt(d)
    o, lse = orc.prefill(q, k, v, scale, causal=causal, softcap=softcap, mask=mask, max_bias=max_bias)
    ob, lb = brute.prefill_decimal(q.tolist(), k.tolist(), v.tolist(), scale, causal, softcap,
                                   None, mask.tolist(), slopes)
    ob = np.array([[[[float(x) for x in row] for row in hh] for hh in ii] for ii in ob])
    lb = np.array([[[(-math.inf if x is None else float(x)) for x in r] for r in hh] for hh in lb])
    _close(o, ob, 1e-12, "masked o vs decimal brute force")
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse)), "masked lse -inf pattern differs from brute force"
    _close(lse[fin], lb[fin], 1e-12, "masked lse vs decimal brute force")


def pin_brute_mask_alibi(orc):
    """Additive mask after the softcap, per-head mask, ALiBi slopes of a 2-head model
    (2^-4, 2^-8 for a maximum bias of 8), GQA, causal on top."""
    _brute_mask_compare(orc, 1, 4, 6, 2, 1, 3, 1, 2, 1.5, True, 8.0, [2.0 ** -4, 2.0 ** -8], 61)


def pin_brute_mask_broadcast(orc):
    """One mask shared by both batches (MB = 1) and by both heads (MH = 1)."""
    _brute_mask_compare(orc, 2, 3, 5, 2, 2, 4, 1, 1, 0.0, False, 0.0, None, 62)
    _brute_mask_compare(orc, 2, 3, 5, 2, 2, 4, 2, 1, 0.0, False, 0.0, None, 63)


def pin_mask_as_causal(orc):
    """A mask of 0 on and below the bottom-right diagonal and -inf above it is the causal mask."""
    rng = _rng(64)
    B, Sq, Sk = 2, 5, 9
    q = _rand(rng, B, Sq, 2, 4)
    k = _rand(rng, B, Sk, 2, 4)
    v = _rand(rng, B, Sk, 2, 3)
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    mask = np.where(j <= i + (Sk - Sq), 0.0, -np.inf)[None, None]
    o1, l1 = orc.prefill(q, k, v, 0.4, causal=True)
    o2, l2 = orc.prefill(q, k, v, 0.4, mask=mask)
    _close(o1, o2, 1e-14, "causal as a mask")
    _close(l1, l2, 1e-14, "lse of causal as a mask")


def pin_mask_constant_shift(orc):
    """Adding c to every mask entry shifts every score of head h by slope_h * c: the
    output is unchanged and lse moves by slope_h * c (softmax shift invariance)."""
    rng = _rng(65)
    Hq = 4
    q = _rand(rng, 1, 3, Hq, 4)
    k = _rand(rng, 1, 6, 2, 4)
    v = _rand(rng, 1, 6, 2, 5)
    mask = _rand(rng, 1, Hq, 3, 6)
    c = 1.75
    slopes = [2.0 ** -2, 2.0 ** -4, 2.0 ** -6, 2.0 ** -8]   # 4 heads, maximum bias 8
    o1, l1 = orc.prefill(q, k, v, 0.5, mask=mask, max_bias=8.0)
    o2, l2 = orc.prefill(q, k, v, 0.5, mask=mask + c, max_bias=8.0)
    _close(o1, o2, 1e-13, "output under a constant mask shift")
    _close(l2 - l1, np.broadcast_to(np.array(slopes)[None, :, None] * c, l1.shape), 1e-13, "lse shift")


def pin_mask_all_neg_inf(orc):
    """A query row whose mask is -inf everywhere sees no key: o = 0 and lse = -inf."""
    rng = _rng(66)
    q = _rand(rng, 1, 3, 1, 4)
    k = _rand(rng, 1, 5, 1, 4)
    v = _rand(rng, 1, 5, 1, 3)
    mask = np.zeros((1, 1, 3, 5))
    mask[0, 0, 1, :] = -np.inf
    o, lse = orc.prefill(q, k, v, 0.5, mask=mask)
    assert np.array_equal(o[0, 1, 0], np.zeros(3)), "fully masked row must be 0"
    assert lse[0, 0, 1] == -np.inf, "fully masked row has lse -inf"
    assert np.isfinite(lse[0, 0, [0, 2]]).all()



# ---------------------------------------------------------------- MLA tail (out-absorb, o-projection)
def pin_mla_tail_hand_example(orc):
    """One token, two heads, latent width 3, v_head_dim 2, hidden 2, worked by hand
    ("MLA Decode Attention Kernel API Reference" page, out_absorb_w [n_heads,
    v_head_dim, kv_lora_rank] and o_proj_w [n_heads * v_head_dim, hidden]):
        head 0: o = (1, 2, 0),  W = [[1, 0, 1], [0, 1, 0]]   -> u = (1, 2)
        head 1: o = (0, 1, -1), W = [[0, 3, 0], [1, 0, -1]]  -> u = (3, 1)
        rows of w_o, head-major: (1, 0), (0, 1), (1, 1), (2, -1)
        y = 1*(1, 0) + 2*(0, 1) + 3*(1, 1) + 1*(2, -1) = (6, 4)"""
    o_lat = np.array([[[1.0, 2.0, 0.0], [0.0, 1.0, -1.0]]])
    w_abs = np.array([[[1.0, 0.0, 1.0], [0.0, 1.0, 0.0]], [[0.0, 3.0, 0.0], [1.0, 0.0, -1.0]]])
    w_o = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [2.0, -1.0]])
    y, u = orc.mla_tail(o_lat, w_abs, w_o)
    _close(u, [[[1.0, 2.0], [3.0, 1.0]]], 0.0, "hand example u")
    _close(y, [[6.0, 4.0]], 0.0, "hand example y")


def pin_mla_tail_identity_absorb(orc):
    """With v_head_dim equal to the latent width and every head's out-absorb the
    identity, u is the attention output itself and the tail is one plain matrix
    product of the tokens' concatenated heads with w_o (numpy's matmul)."""
    rng = _rng(70)
    T, H, R, N = 3, 4, 8, 5
    o_lat = _rand(rng, T, H, R)
    w_abs = np.broadcast_to(np.eye(R), (H, R, R)).copy()
    w_o = _rand(rng, H * R, N)
    y, u = orc.mla_tail(o_lat, w_abs, w_o)
    _close(u, o_lat, 0.0, "identity absorb gives u = o")
    _close(y, np.matmul(o_lat.reshape(T, H * R), w_o), 1e-12, "identity absorb gives one matmul")


def pin_mla_tail_head_rescale(orc):
    """Scaling head h's out-absorb by s_h and its rows of w_o by 1 / s_h leaves y
    unchanged and scales u[:, h] by s_h: each head's value block meets its own
    o-projection rows (bilinearity of the two products)."""
    rng = _rng(71)
    T, H, R, DV, N = 2, 3, 6, 4, 7
    o_lat = _rand(rng, T, H, R)
    w_abs = _rand(rng, H, DV, R)
    w_o = _rand(rng, H * DV, N)
    s = np.array([2.0, -0.5, 4.0])
    y1, u1 = orc.mla_tail(o_lat, w_abs, w_o)
    y2, u2 = orc.mla_tail(o_lat, w_abs * s[:, None, None], w_o / np.repeat(s, DV)[:, None])
    _close(y1, y2, 1e-12, "y under per-head rescaling")
    _close(u2, u1 * s[None, :, None], 1e-12, "u scales with its head")


PINS = {name[4:]: fn for name, fn in sorted(globals().items()) if name.startswith("pin_") and callable(fn)}
