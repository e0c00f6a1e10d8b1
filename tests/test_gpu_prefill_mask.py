"""GPU parity of attn_prefill_fwd_ex with an additive fp16 mask and ALiBi slopes against the
fp64 CPU oracle, through the C ABI."""

import math

import numpy as np
import pytest
import torch

import oracle
from attention_flash_attn_amd import binding, synth
from gpu_util import check_close, dev, dev_bf16, host

pytestmark = pytest.mark.gpu

LSE_TOL = -math.log(1 - 2.0 ** -8) + 1e-5   # bf16-rounded probabilities, as for the unmasked path


def check_masked(B, Sq, Sk, Hq, Hkv, dk, dv, MB, MH, kind="random", width=None, causal=False, softcap=0.0,
                 sinks=False, max_bias=0.0, o_dtype="f32", std=1.0, seed=300, mask=None):
    print("masked case B=%d Sq=%d Sk=%d Hq=%d Hkv=%d d=%d/%d mask=[%d,%d,%s,%s] causal=%d softcap=%g sinks=%d "
          "max_bias=%g %s" % (B, Sq, Sk, Hq, Hkv, dk, dv, MB, MH, kind, width, causal, softcap, sinks, max_bias,
                              o_dtype), flush=True)
    case = synth.prefill_case(seed, B, Sq, Sk, Hq, Hkv, dk, dv, std=std, sinks=sinks)
    if mask is None:
        mask = synth.mask_case(seed, MB, MH, Sq, Sk, width=width, kind=kind)
    scale = 1.0 / math.sqrt(dk)
    q, k, v = dev_bf16(case["q"]), dev_bf16(case["k"]), dev_bf16(case["v"])
    o = torch.empty((B, Sq, Hq, dv), device="cuda", dtype=torch.float32 if o_dtype == "f32" else torch.bfloat16)
    lse = torch.empty((B, Hq, Sq), device="cuda", dtype=torch.float32)
    sk = dev(case["sinks"]) if case["sinks"] is not None else None
    binding.attn_prefill_fwd_ex(q, k, v, o, lse, scale=scale, causal=causal, softcap=softcap, sinks=sk,
                                mask=dev(mask), max_bias=max_bias)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(case["q"], case["k"], case["v"], scale, causal=causal, softcap=softcap,
                            sinks=case["sinks"], mask=mask, max_bias=max_bias)
    check_close(host(o), ro, o_dtype, "o")
    got_l = host(lse)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(got_l), fin), "lse -inf pattern"
    if fin.any():
        assert np.abs(got_l[fin] - rl[fin]).max() < LSE_TOL
    return host(o), got_l


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 32), (64, 64), (96, 96), (128, 128), (192, 192), (256, 256),
                                   (192, 128)])
def test_mask_head_dims(dk, dv):
    check_masked(1, 150, 170, 2, 1, dk, dv, 1, 2, seed=301)
    check_masked(1, 97, 97, 2, 2, dk, dv, 1, 1, causal=True, o_dtype="bf16", seed=302)


def test_mask_per_batch_and_head_gqa():
    check_masked(2, 200, 200, 4, 2, 128, 128, 2, 4, seed=303)
    check_masked(2, 77, 140, 8, 2, 64, 64, 1, 8, causal=True, o_dtype="bf16", seed=304)
    check_masked(3, 64, 64, 4, 4, 64, 64, 3, 1, seed=305)                 # per batch, shared by heads


def test_mask_row_stride_wider_than_keys():
    check_masked(1, 129, 190, 4, 1, 256, 256, 1, 4, width=196, softcap=20.0, sinks=True, o_dtype="bf16",
                 std=0.5, seed=306)
    check_masked(1, 100, 61, 2, 1, 128, 128, 1, 1, width=128, seed=307)


def test_alibi_distance_mask():
    # 12 heads (not a power of two: the m1 branch of the slope schedule), mask carries causality
    check_masked(1, 300, 300, 12, 4, 128, 128, 1, 1, kind="distance", max_bias=8.0, seed=308)
    # Sq < Sk (bottom-right positions), d = 64, bf16 output, with the causal flag on as well
    check_masked(2, 90, 250, 8, 8, 64, 64, 1, 1, kind="distance", max_bias=8.0, causal=True, o_dtype="bf16",
                 seed=309)
    check_masked(1, 64, 64, 4, 1, 256, 256, 1, 1, kind="distance", max_bias=4.0, seed=310)


def test_mask_fully_masked_rows():
    Sq, Sk = 70, 90
    mask = synth.mask_case(311, 1, 1, Sq, Sk)
    mask[0, 0, 5, :] = -np.inf
    mask[0, 0, 66, :] = -np.inf
    o, lse = check_masked(1, Sq, Sk, 2, 1, 128, 128, 1, 1, seed=311, mask=mask)
    assert np.array_equal(o[0, [5, 66]], np.zeros((2, 2, 128)))
    assert np.all(lse[0, :, [5, 66]] == -np.inf)


def test_zero_mask_matches_unmasked():
    """A mask of zeros changes nothing: both calls agree with the unmasked oracle."""
    case = synth.prefill_case(312, 1, 256, 256, 4, 2, 128, 128)
    q, k, v = dev_bf16(case["q"]), dev_bf16(case["k"]), dev_bf16(case["v"])
    o1 = torch.empty((1, 256, 4, 128), device="cuda", dtype=torch.float32)
    o2 = torch.empty_like(o1)
    binding.attn_prefill_fwd(q, k, v, o1, scale=0.1, causal=True)
    mask = torch.zeros((1, 1, 256, 256), device="cuda", dtype=torch.float16)
    binding.attn_prefill_fwd_ex(q, k, v, o2, scale=0.1, causal=True, mask=mask)
    torch.cuda.synchronize()
    ref, _ = oracle.prefill(case["q"], case["k"], case["v"], 0.1, causal=True)
    check_close(host(o1), ref, "f32", "unmasked")
    check_close(host(o2), ref, "f32", "zero mask")
