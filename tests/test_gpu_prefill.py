"""GPU parity of attn_prefill_fwd against the fp64 CPU oracle (through the C ABI)."""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from attention_flash_attn_amd import binding, synth
from gpu_util import check_close, dev, dev_bf16, host, prefill_value_range, spread_bound

pytestmark = pytest.mark.gpu

LSE_TOL = -math.log(1 - 2.0 ** -8) + 1e-5


def run_prefill(case, scale, causal, softcap, o_dtype, with_lse=True):
    q, k, v = dev_bf16(case["q"]), dev_bf16(case["k"]), dev_bf16(case["v"])
    B, Sq, Hq, dk = q.shape
    dv = v.shape[3]
    o = torch.empty((B, Sq, Hq, dv), device="cuda", dtype=torch.float32 if o_dtype == "f32" else torch.bfloat16)
    lse = torch.empty((B, Hq, Sq), device="cuda", dtype=torch.float32) if with_lse else None
    sinks = dev(case["sinks"]) if case["sinks"] is not None else None
    binding.attn_prefill_fwd(q, k, v, o, lse, scale=scale, causal=causal, softcap=softcap, sinks=sinks)
    torch.cuda.synchronize()
    return o, lse


def check_case(B, Sq, Sk, Hq, Hkv, dk, dv, causal=False, softcap=0.0, sinks=False, o_dtype="f32", std=1.0,
               seed=100):
    print("case B=%d Sq=%d Sk=%d Hq=%d Hkv=%d dk=%d dv=%d causal=%d softcap=%g sinks=%d %s" %
          (B, Sq, Sk, Hq, Hkv, dk, dv, causal, softcap, sinks, o_dtype), flush=True)
    case = synth.prefill_case(seed, B, Sq, Sk, Hq, Hkv, dk, dv, std=std, sinks=sinks)
    scale = 1.0 / math.sqrt(dk)
    o, lse = run_prefill(case, scale, causal, softcap, o_dtype)
    ro, rl = oracle.prefill(case["q"], case["k"], case["v"], scale, causal=causal, softcap=softcap,
                            sinks=case["sinks"])
    bound = None
    if std > 1.0:  # more than unit spread: the bar derived from the arithmetic
        vmax, vmin = prefill_value_range(synth.bf16_bits_to_f32(case["v"]), Sq, Hq, causal)
        bound = spread_bound(ro, vmax, vmin, Sk, float(np.abs(synth.bf16_bits_to_f32(case["v"])).max()))
    check_close(host(o), ro, o_dtype, "o", bound=bound)
    got_l = host(lse)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(got_l), fin)
    if fin.any():
        # The kernel sums the bf16-rounded probabilities. bf16 keeps 8 significand bits, so
        # round-to-nearest has relative error <= 2^-8 per probability, the normaliser is
        # Z' = Z (1 + d) with |d| <= 2^-8 (reached when one probability dominates) and
        # |ln Z' - ln Z| <= -ln(1 - 2^-8) = 3.914e-3; fp32 score and exp2/log2 errors add
        # well under 1e-5.
        assert np.abs(got_l[fin] - rl[fin]).max() < LSE_TOL


def test_config1_single_head_d16():
    c = synth.CONFIGS["c1_single_head_d16"]
    case = synth.prefill_case(c["seed"], c["B"], c["Sq"], c["Sk"], c["Hq"], c["Hkv"], c["dk"], c["dv"])
    o, lse = run_prefill(case, c["scale"], False, 0.0, "f32")
    ro, rl = oracle.prefill(case["q"], case["k"], case["v"], c["scale"])
    err, cos = check_close(host(o), ro, "f32", "config 1")
    print("config 1: max abs err %.3g cosine %.8f" % (err, cos))


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 32), (64, 64), (96, 96), (128, 128), (192, 192), (256, 256),
                                   (192, 128)])
def test_head_dims(dk, dv):
    check_case(1, 200, 200, 2, 1, dk, dv, causal=False, o_dtype="f32")
    check_case(1, 131, 131, 2, 2, dk, dv, causal=True, o_dtype="bf16", seed=101)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (8, 1), (16, 2)])
def test_gqa_and_tails(Hq, Hkv):
    check_case(2, 77, 77, Hq, Hkv, 64, 64, causal=True, o_dtype="f32", seed=102)
    check_case(1, 300, 257, Hq, Hkv, 128, 128, causal=False, o_dtype="bf16", seed=103)


def test_causal_gqa_grouped_xcd_order():
    """Causal GQA with B * Hkv a multiple of 8: workgroups are ordered by KV group."""
    check_case(2, 600, 600, 16, 4, 128, 128, causal=True, o_dtype="bf16", seed=115)
    check_case(1, 300, 300, 16, 8, 256, 256, causal=True, sinks=True, o_dtype="f32", std=0.5, seed=116)


def test_causal_rectangular_bottom_right():
    check_case(1, 70, 333, 2, 1, 128, 128, causal=True, o_dtype="f32", seed=104)   # Sq < Sk
    check_case(1, 200, 60, 2, 1, 64, 64, causal=True, o_dtype="f32", seed=105)     # Sq > Sk: empty rows


def test_softcap_and_sinks():
    check_case(1, 256, 256, 4, 2, 128, 128, causal=True, softcap=5.0, sinks=True, o_dtype="f32", seed=106)
    check_case(1, 129, 190, 4, 1, 256, 256, causal=False, softcap=0.0, sinks=True, o_dtype="bf16", std=0.5,
               seed=107)
    check_case(1, 64, 64, 2, 2, 64, 64, causal=True, softcap=0.5, sinks=True, o_dtype="f32", std=3.0, seed=108)


def test_single_query_and_single_key():
    check_case(1, 1, 1, 1, 1, 64, 64, causal=True, o_dtype="f32", seed=109)
    check_case(3, 1, 500, 2, 1, 128, 128, causal=True, o_dtype="f32", seed=110)


def test_bitwise_repeatable():
    case = synth.prefill_case(111, 1, 384, 384, 4, 2, 128, 128)
    o1, _ = run_prefill(case, 0.088, True, 0.0, "bf16")
    o2, _ = run_prefill(case, 0.088, True, 0.0, "bf16")
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def _full_config(name):
    """Every output element of a full-size workload against the oracle (all rows, heads and
    batch entries), for the bf16 output the workload specifies and for an fp32 output of
    the same launch configuration (only the store type differs)."""
    c = synth.CONFIGS[name]
    print("full-size %s, every element" % name, flush=True)
    case = synth.prefill_case(c["seed"], c["B"], c["Sq"], c["Sk"], c["Hq"], c["Hkv"], c["dk"], c["dv"],
                              std=c["std"], sinks=c["sinks"])
    o, lse = run_prefill(case, c["scale"], c["causal"], c["softcap"], c["o_dtype"])
    o32 = torch.empty(o.shape, device="cuda", dtype=torch.float32)
    q, k, v = dev_bf16(case["q"]), dev_bf16(case["k"]), dev_bf16(case["v"])
    sinks = dev(case["sinks"]) if case["sinks"] is not None else None
    binding.attn_prefill_fwd(q, k, v, o32, None, scale=c["scale"], causal=c["causal"], softcap=c["softcap"],
                             sinks=sinks)
    torch.cuda.synchronize()
    got, got32, got_l = host(o), host(o32), host(lse)
    del q, k, v, o, o32, lse
    print("oracle on all %d (batch, head) pairs" % (c["B"] * c["Hq"]), flush=True)
    ro, rl = oracle.prefill(case["q"], case["k"], case["v"], c["scale"], causal=c["causal"],
                            softcap=c["softcap"], sinks=case["sinks"])
    e1, c1 = check_close(got, ro, "bf16", name + " bf16")
    e2, c2 = check_close(got32, ro, "f32", name + " f32")
    assert np.abs(got_l - rl).max() < LSE_TOL
    print("%s: %d elements | bf16 max err %.3g cos %.8f | f32 max err %.3g cos %.8f" %
          (name, ro.size, e1, c1, e2, c2))


def test_config2_full_size():
    _full_config("c2_causal_mha_d128")


def test_config3a_full_size():
    _full_config("c3a_gqa_d256")


def test_config3b_full_size():
    _full_config("c3b_gqa_d256_causal_softcap")
