"""Helpers for GPU parity tests: move synthetic inputs to the device, compare with the oracle."""

import numpy as np
import torch

BF16_TOL = 1e-2       # max-abs bound on fp32 outputs (and floor for bf16 outputs)
COS_MIN = 0.99999     # cosine bound


def dev_bf16(bits):
    """uint16 bf16 bit patterns -> bfloat16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda").view(torch.bfloat16)


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def host(t):
    """Device tensor -> float64 numpy."""
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def bf16_ulp(x):
    """Spacing of bf16 at |x| (2^(e-7) for x in [2^e, 2^(e+1)))."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    e = np.floor(np.log2(a))
    return 2.0 ** (e - 7)


def cosine(a, b):
    a = a.ravel()
    b = b.ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


U_BF16 = 2.0 ** -8     # unit roundoff of round-to-nearest bf16 (8 significand bits)
U_F32 = 2.0 ** -24


def spread_bound(ref, vmax, vmin, n_keys, vabs, partials_16bit=False):
    """Per-element bound on |O_gpu - O_ref| implied by the kernels' arithmetic, for
    inputs whose spread is not of unit size.

    The kernels round every probability p_j to bf16 (relative error d_j, |d_j| <= u =
    2^-8) and sum the rounded values in fp32; O = sum p~_j V_j / (sum p~_j + e^sink).
    Then O~ - O = sum_j (p~_j - p_j)(V_j - O) / D~, so
        |O~ - O| <= u / (1 - u) * max_j |V_j - O|
    over the row's live keys (a sink only enlarges D~). max_j |V_j - O| is
    max(vmax - O, O - vmin) with vmax / vmin the element-wise maximum and minimum of
    the row's live values (or of any superset of them). Split-KV partials stored
    normalised in bf16 add u * max(|vmax|, |vmin|) (each partial is a convex
    combination of the values). The fp32 sums over at most n_keys terms add
    2 * n_keys * 2^-24 * vabs (vabs = max |V|), and 1e-6 covers the exp2 and score
    rounding."""
    ref = np.asarray(ref, dtype=np.float64)
    spread = np.maximum(np.maximum(vmax - ref, ref - vmin), 0.0)
    b = U_BF16 / (1.0 - U_BF16) * spread + 2.0 * n_keys * U_F32 * vabs + 1e-6
    if partials_16bit:
        b = b + U_BF16 * np.maximum(np.abs(vmax), np.abs(vmin))
    return b


def prefill_value_range(v, Sq, Hq, causal):
    """Element-wise max / min of the values each query row can see ([B, Sq, Hq, dv]):
    v [B, Sk, Hkv, dv] as floats; causal rows see keys j <= Sk - Sq + i. Rows that see
    no key get 0 (their output is 0)."""
    v = np.asarray(v, dtype=np.float64)
    B, Sk, Hkv, dv = v.shape
    group = Hq // Hkv
    if causal:
        cmax = np.maximum.accumulate(v, axis=1)
        cmin = np.minimum.accumulate(v, axis=1)
        last = np.arange(Sq) + (Sk - Sq)
        idx = np.clip(last, 0, Sk - 1)
        vmax, vmin = cmax[:, idx], cmin[:, idx]
        empty = last < 0
        vmax[:, empty] = 0.0
        vmin[:, empty] = 0.0
    else:
        vmax = np.broadcast_to(v.max(axis=1, keepdims=True), (B, Sq, Hkv, dv))
        vmin = np.broadcast_to(v.min(axis=1, keepdims=True), (B, Sq, Hkv, dv))
    return np.repeat(vmax, group, axis=2), np.repeat(vmin, group, axis=2)


def check_close(got, ref, out_dtype, what="", bound=None):
    """The bar: fp32 output within max-abs 1e-2; bf16 output within
    max(1e-2, one bf16 ulp of the reference) per element; cosine >= 0.99999.

    bound (optional, per element, from spread_bound): for inputs of more than unit
    spread the absolute bar becomes max(1e-2, bound) (bf16 outputs: plus one ulp of the
    reference for the final rounding). The five benchmark workloads use the plain bar."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), "%s: non-finite output" % what
    err = np.abs(got - ref)
    tol = BF16_TOL if bound is None else np.maximum(BF16_TOL, bound)
    if out_dtype == "f32":
        bad = err > tol
        assert not bad.any(), "%s: max abs err %.4g (%d elements beyond the bar)" % (what, err.max(), bad.sum())
    else:
        lim = np.maximum(tol, bf16_ulp(ref)) if bound is None else np.maximum(BF16_TOL, bound + bf16_ulp(ref))
        bad = err > lim
        assert not bad.any(), "%s: %d elements beyond bound, worst err %.4g" % (what, bad.sum(), err.max())
    c = cosine(got, ref)
    if np.abs(ref).max() > 0:
        assert c >= COS_MIN, "%s: cosine %.7f" % (what, c)
    return float(err.max()), c
