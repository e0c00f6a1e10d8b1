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


def check_close(got, ref, out_dtype, what="", vscale=1.0):
    """The bar: fp32 output within max-abs 1e-2; bf16 output within
    max(1e-2, one bf16 ulp of the reference) per element; cosine >= 0.99999.

    The 1e-2 is set for values of unit spread. The output is linear in V, and its main
    error, the rounding of each probability to bf16 (relative 2^-9, so at most
    2^-9 max_j |V_j - O| per element), grows with V's spread: for values of standard
    deviation s > 1 (vscale) the absolute bar is 1e-2 * s."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), "%s: non-finite output" % what
    err = np.abs(got - ref)
    tol = BF16_TOL * max(1.0, vscale)
    if out_dtype == "f32":
        assert err.max() <= tol, "%s: max abs err %.4g" % (what, err.max())
    else:
        bound = np.maximum(tol, bf16_ulp(ref))
        bad = err > bound
        assert not bad.any(), "%s: %d elements beyond bound, worst err %.4g" % (what, bad.sum(), err.max())
    c = cosine(got, ref)
    if np.abs(ref).max() > 0:
        assert c >= COS_MIN, "%s: cosine %.7f" % (what, c)
    return float(err.max()), c
