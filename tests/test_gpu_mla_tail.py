"""GPU parity of attn_mla_tail (out-absorb + o-projection after MLA decode) against the
fp64 oracle, through the C ABI.

Bars:
  * integer-valued inputs whose every intermediate is exact in bf16 / fp32 (|u| <= 256,
    |y| < 2^24): the result must equal the oracle bit for bit (fp32 output);
  * random inputs: per element |y - y_ref| <= 2^-8 * y_abs + 2^-8 * |y_ref|, where y_abs
    is the oracle run on the absolute values of every input. u is rounded to bf16
    (relative error <= 2^-9), the two fp32 sums add at most 512 * 2^-24 and
    K * 2^-24 <= 2^-10 (K <= 16384) of the absolute sums, and a bf16 output adds 2^-9
    of |y|, all below those two terms; plus relative RMS error <= 2^-8 and cosine
    >= 0.99999 (rounding errors are independent, so the RMS is near 2^-9 / sqrt(3)).
"""

import numpy as np
import pytest
import torch

import oracle
from attention_flash_attn_amd import binding, synth
from gpu_util import COS_MIN, cosine, dev_bf16, host

pytestmark = pytest.mark.gpu


def run_tail(o_lat, w_abs, w_o, y_dtype):
    T, H, R = o_lat.shape
    N = w_o.shape[1]
    DV = w_abs.shape[1]
    y = torch.empty((T, N), device="cuda", dtype=torch.float32 if y_dtype == "f32" else torch.bfloat16)
    ws = torch.empty(binding.attn_mla_tail_workspace_bytes(T, H, R, DV, N), device="cuda", dtype=torch.uint8)
    binding.attn_mla_tail(dev_bf16(o_lat), dev_bf16(w_abs), dev_bf16(w_o), y, ws)
    torch.cuda.synchronize()
    return y


def int_bf16(rng, shape, lo, hi, p_zero=0.0):
    """Integer values in [lo, hi] (some set to zero) as bf16 bit patterns (exact)."""
    x = rng.integers(lo, hi, size=shape, endpoint=True).astype(np.float32)
    if p_zero:
        x[rng.random(shape) < p_zero] = 0.0
    return synth.to_bf16_bits(x)


@pytest.mark.parametrize("T,H,R,DV,N", [(5, 4, 128, 32, 256), (37, 8, 256, 32, 384), (70, 4, 128, 64, 128),
                                        (1, 2, 128, 64, 128)])
def test_tail_exact_integers(T, H, R, DV, N):
    print("mla tail exact T=%d H=%d R=%d DV=%d N=%d" % (T, H, R, DV, N), flush=True)
    rng = np.random.Generator(np.random.PCG64([T, H, R, DV, N]))
    o_lat = int_bf16(rng, (T, H, R), -1, 1)
    w_abs = int_bf16(rng, (H, DV, R), -1, 1)
    w_o = int_bf16(rng, (H * DV, N), -1, 1, p_zero=0.5)
    y_ref, u_ref = oracle.mla_tail(o_lat, w_abs, w_o)
    assert np.abs(u_ref).max() <= 256 and np.abs(y_ref).max() < 2 ** 24
    y = host(run_tail(o_lat, w_abs, w_o, "f32"))
    assert np.array_equal(y, y_ref), "max err %g" % np.abs(y - y_ref).max()


def check_tail(case, y_dtype, what):
    o_lat, w_abs, w_o = case["o_lat"], case["w_absorb"], case["w_o"]
    y = host(run_tail(o_lat, w_abs, w_o, y_dtype))
    y_ref, _ = oracle.mla_tail(o_lat, w_abs, w_o)
    absb = lambda b: synth.to_bf16_bits(np.abs(synth.bf16_bits_to_f32(b)))
    y_abs, _ = oracle.mla_tail(absb(o_lat), absb(w_abs), absb(w_o))
    err = np.abs(y - y_ref)
    bound = 2.0 ** -8 * y_abs + 2.0 ** -8 * np.abs(y_ref)
    assert np.isfinite(y).all(), what
    assert (err <= bound).all(), "%s: %d elements beyond the bound, worst ratio %.3g" % (
        what, (err > bound).sum(), (err / bound).max())
    rel = np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)
    assert rel <= 2.0 ** -8, "%s: relative RMS error %.3g" % (what, rel)
    assert cosine(y, y_ref) >= COS_MIN, what
    return y, rel


@pytest.mark.parametrize("T,H,R,DV,N,y_dtype", [(16, 16, 512, 128, 1024, "bf16"), (3, 8, 256, 64, 384, "f32"),
                                                (50, 4, 128, 32, 256, "bf16")])
def test_tail_random(T, H, R, DV, N, y_dtype):
    print("mla tail random T=%d H=%d R=%d DV=%d N=%d %s" % (T, H, R, DV, N, y_dtype), flush=True)
    check_tail(synth.mla_tail_case(400 + T, T, H, R, DV, N), y_dtype, "random tail")


def test_tail_full_size():
    """16 tokens x 128 heads, latent 512, v_head_dim 128, hidden 7168 (all of y checked)."""
    c = synth.MLA_TAIL
    print("mla tail full size %s" % c, flush=True)
    case = synth.mla_tail_case(c["seed"], c["T"], c["H"], c["R"], c["DV"], c["N"])
    _, rel = check_tail(case, "bf16", "full-size tail")
    print("full-size tail: relative RMS error %.3g" % rel)


def test_tail_repeatable():
    """Fixed slice order: two calls give identical bits."""
    case = synth.mla_tail_case(410, 16, 16, 512, 128, 1024)
    y1 = run_tail(case["o_lat"], case["w_absorb"], case["w_o"], "bf16")
    y2 = run_tail(case["o_lat"], case["w_absorb"], case["w_o"], "bf16")
    assert torch.equal(y1, y2)
