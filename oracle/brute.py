"""Scalar brute force of the attention definition in 40-digit decimal arithmetic.

TEST INFRASTRUCTURE: pins the fp64 oracle on tiny inputs. It is written
independently of oracle.py (pure Python loops, decimal.Decimal, its own exp and
tanh handling) so that a slip in the vectorised oracle (a transposed operand,
a wrong head map, a dropped term) shows up as a mismatch.

Definition followed (the score step and final normalisation of the tensor
kernel on the "ggml-metal: FA tensor path: gate to the (256, 256) shape" page;
the unscaled-product lesson of the "UMMA FMHA" page): for every query row,
score each visible key by scale * dot(q, k), cap it with softcap * tanh(s /
softcap) when softcap is non-zero, exponentiate against the largest term, add
the head's sink as a value-less term, and divide the weighted value sum by the
total. tanh is taken from exponentials: tanh(y) = (e^{2y} - 1) / (e^{2y} + 1).
"""

from decimal import Decimal, getcontext

getcontext().prec = 40

__all__ = ["attention_rows_decimal", "prefill_decimal"]


def _d(x):
    return Decimal(float(x))


def _tanh(y):
    e2 = (2 * y).exp()
    return (e2 - 1) / (e2 + 1)


def attention_rows_decimal(qrows, keys, values, scale, softcap=0.0, sink=None, visible=None, add=None):
    """qrows: list of R lists (dk); keys: list of N lists (dk); values: list of N lists (dv).
    visible(r, j) -> bool or None; add(r, j) -> float (an additive score term applied
    after the softcap; -inf hides the key) or None. Returns (o as list of lists of
    Decimal, lse list)."""
    sc = _d(scale)
    cap = _d(softcap)
    outs, lses = [], []
    for r, qr in enumerate(qrows):
        terms = []  # (score, value row or None)
        for j, kr in enumerate(keys):
            if visible is not None and not visible(r, j):
                continue
            s = Decimal(0)
            for a, b in zip(qr, kr):
                s += _d(a) * _d(b)
            s = s * sc
            if cap != 0:
                s = cap * _tanh(s / cap)
            if add is not None:
                extra = float(add(r, j))
                if extra == float("-inf"):
                    continue
                s = s + _d(extra)
            terms.append((s, values[j]))
        n_live = len(terms)
        if sink is not None:
            terms.append((_d(sink), None))
        dv = len(values[0]) if values else 0
        if not terms:
            outs.append([Decimal(0)] * dv)
            lses.append(None)  # -inf
            continue
        big = max(t[0] for t in terms)
        total = Decimal(0)
        acc = [Decimal(0)] * dv
        for s, vr in terms:
            w = (s - big).exp()
            total += w
            if vr is not None:
                for d in range(dv):
                    acc[d] += w * _d(vr[d])
        if n_live == 0:
            outs.append([Decimal(0)] * dv)
        else:
            outs.append([a / total for a in acc])
        lses.append(big + total.ln())
    return outs, lses


def prefill_decimal(q, k, v, scale, causal=False, softcap=0.0, sinks=None, mask=None, slopes=None):
    """q [B][Sq][Hq][dk], k [B][Sk][Hkv][dk], v [B][Sk][Hkv][dv] as nested lists of floats.
    mask [MB][MH][Sq][Sk] (nested lists, may hold -inf) is added to head h of batch b
    as slopes[h] * mask[b % MB][h % MH] (slopes given explicitly; 1 when None).
    Returns o [B][Sq][Hq][dv] and lse [B][Hq][Sq] (None for -inf), all Decimal."""
    B, Sq, Hq = len(q), len(q[0]), len(q[0][0])
    Sk, Hkv = len(k[0]), len(k[0][0])
    per = Hq // Hkv
    o = [[[None] * Hq for _ in range(Sq)] for _ in range(B)]
    lse = [[[None] * Sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // per
            qrows = [q[b][i][h] for i in range(Sq)]
            keys = [k[b][j][g] for j in range(Sk)]
            vals = [v[b][j][g] for j in range(Sk)]
            vis = None
            if causal:
                off = Sk - Sq
                vis = (lambda r, j, off=off: j <= r + off)
            sink = None if sinks is None else sinks[h]
            add = None
            if mask is not None:
                mrow = mask[b % len(mask)][h % len(mask[0])]
                sl = 1.0 if slopes is None else slopes[h]
                add = (lambda r, j, mrow=mrow, sl=sl:
                       float("-inf") if mrow[r][j] == float("-inf") else sl * mrow[r][j])
            ob, lb = attention_rows_decimal(qrows, keys, vals, scale, softcap, sink, vis, add)
            for i in range(Sq):
                o[b][i][h] = ob[i]
                lse[b][h][i] = lb[i]
    return o, lse
