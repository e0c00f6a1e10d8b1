"""attn_decode_fwd_noalloc (static per-GPU scratch, no workspace argument) against
attn_decode_fwd (caller's workspace) through the C ABI: the same kernels on the same
inputs, so the outputs must be bit-identical, and both within the parity bar of the
oracle. Two calls in a row per mode, the second with a smaller input (the scratch keeps
the first call's contents)."""

import math

import numpy as np
import pytest
import torch

import oracle
from attention_flash_attn_amd import binding, synth
from gpu_util import check_close, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def _paged_pair(seed, B, Hq, Hkv, d, lo, hi, Sq=1, causal=False):
    print("no-alloc paged B=%d Hq=%d Hkv=%d d=%d len[%d,%d] Sq=%d" % (B, Hq, Hkv, d, lo, hi, Sq), flush=True)
    case = synth.paged_case(seed, B, Hq, Hkv, d, d, lo, hi, Sq=Sq)
    q, kc, vc = dev_bf16(case["q"]), dev_bf16(case["k_cache"]), dev_bf16(case["v_cache"])
    table, lens = dev(case["block_table"]), dev(case["seq_lens"])
    scale = 1.0 / math.sqrt(d)
    o_ws = torch.empty((B, Sq, Hq, d), device="cuda", dtype=torch.bfloat16)
    o_na = torch.full_like(o_ws, float("nan"))
    ws = torch.empty(binding.attn_decode_workspace_bytes(B, Hq, Hkv, Sq, hi, d, d), device="cuda", dtype=torch.uint8)
    binding.attn_decode_fwd(q, kc, vc, o_ws, ws, scale=scale, Sk_max=hi, causal=causal, block_table=table,
                            seq_lens=lens)
    binding.attn_decode_fwd_noalloc(q, kc, vc, o_na, scale=scale, Sk_max=hi, causal=causal, block_table=table,
                                    seq_lens=lens)
    torch.cuda.synchronize()
    assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16)), "no-alloc output differs from workspace output"
    ro, _ = oracle.decode_paged(case["q"], case["k_cache"], case["v_cache"], case["block_table"], case["seq_lens"],
                                scale, causal=causal)
    check_close(host(o_na), ro, "bf16", "no-alloc paged decode")


def _gathered_pair(seed, T, Hq, n_rows, n_sel):
    print("no-alloc gathered T=%d Hq=%d n_sel=%d" % (T, Hq, n_sel), flush=True)
    case = synth.gathered_case(seed, T, Hq, 576, 512, n_rows, n_sel, row_dim=576, future_keys=min(16, n_sel))
    kv = dev_bf16(case["kv"])
    q = dev_bf16(case["q"]).view(T, 1, Hq, 576)
    ri, kp, qp = dev(case["row_index"]), dev(case["key_pos"]), dev(case["q_pos"])
    o_ws = torch.empty((T, 1, Hq, 512), device="cuda", dtype=torch.float32)
    o_na = torch.full_like(o_ws, float("nan"))
    ws = torch.empty(binding.attn_decode_workspace_bytes(T, Hq, 1, 1, n_sel, 576, 512), device="cuda",
                     dtype=torch.uint8)
    kw = dict(scale=1.0 / 24, Sk_max=n_sel, causal=True, row_index=ri, key_pos=kp, q_pos=qp, dk=576, dv=512)
    binding.attn_decode_fwd(q, kv[:, :576], kv[:, :512], o_ws, ws, **kw)
    binding.attn_decode_fwd_noalloc(q, kv[:, :576], kv[:, :512], o_na, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_ws.view(torch.int32), o_na.view(torch.int32)), "no-alloc output differs from workspace output"
    ro, _ = oracle.decode_gathered(case["q"], case["kv"], case["kv"][:, :512], case["row_index"], case["key_pos"],
                                   case["q_pos"], 1.0 / 24, causal=True)
    check_close(host(o_na[:, 0]), ro, "f32", "no-alloc gathered decode")


def test_noalloc_paged_two_calls_second_smaller():
    _paged_pair(501, 16, 32, 4, 128, 1000, 6000, Sq=2, causal=True)
    _paged_pair(502, 3, 8, 2, 64, 10, 700)


def test_noalloc_gathered_two_calls_second_smaller():
    c = synth.CONFIGS["c5_gathered_mla_decode"]
    _gathered_pair(c["seed"], c["T"], c["Hq"], c["n_rows"], c["n_sel"])   # the full workload shape
    _gathered_pair(503, 2, 20, 4096, 300)


def test_noalloc_rejects_past_the_scratch_and_leaves_outputs():
    """A call that needs more than the static scratch is refused with ATTN_ERR_UNSUPPORTED
    and enqueues nothing (the output keeps its contents)."""
    B, Hq, Hkv, Sq, hi, d = 256, 64, 8, 8, 32768, 128
    assert binding.attn_decode_workspace_bytes(B, Hq, Hkv, Sq, hi, d, d) > (64 << 20)
    q = torch.zeros((B, Sq, Hq, d), device="cuda", dtype=torch.bfloat16)
    kc = torch.zeros((4, Hkv, 64, d), device="cuda", dtype=torch.bfloat16)
    o = torch.full((B, Sq, Hq, d), 7.0, device="cuda", dtype=torch.bfloat16)
    table = torch.zeros((B, 512), device="cuda", dtype=torch.int32)
    lens = torch.zeros((B,), device="cuda", dtype=torch.int32)
    with pytest.raises(binding.AttnError) as ei:
        binding.attn_decode_fwd_noalloc(q, kc, kc, o, scale=0.1, Sk_max=hi, block_table=table, seq_lens=lens)
    assert ei.value.status == binding.ATTN_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
