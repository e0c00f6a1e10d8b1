"""GPU parity for the other operand types: fp16 K/V, fp32 and fp16 Q (prefill, paged and
gathered decode), against the fp64 oracle on the same values."""

import math

import numpy as np
import pytest
import torch

import oracle
from attention_flash_attn_amd import binding, synth
from gpu_util import check_close, dev, host

pytestmark = pytest.mark.gpu

LSE_TOL = -math.log(1 - 2.0 ** -8) + 1e-5   # bf16-rounded probabilities (fp16 ones are finer)


def to_dev(a):
    """uint16 arrays are bf16 bit patterns; float16 / float32 arrays go as they are."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(a).to("cuda")


def prefill_case(seed, B, Sq, Sk, Hq, Hkv, dk, dv, qt, kvt, std=1.0):
    q = synth.normal_typed(seed, 0, (B, Sq, Hq, dk), qt, std)
    k = synth.normal_typed(seed, 1, (B, Sk, Hkv, dk), kvt, std)
    v = synth.normal_typed(seed, 2, (B, Sk, Hkv, dv), kvt, std)
    return q, k, v


@pytest.mark.parametrize("qt,kvt", [("f16", "f16"), ("f32", "f16"), ("bf16", "f16"), ("f32", "bf16"),
                                    ("f16", "bf16")])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (256, 256), (192, 128)])
def test_prefill_operand_types(qt, kvt, dk, dv):
    print("prefill q=%s kv=%s d=%d/%d" % (qt, kvt, dk, dv), flush=True)
    B, Sq, Sk, Hq, Hkv = 1, 150, 170, 4, 2
    q, k, v = prefill_case(400 + dk, B, Sq, Sk, Hq, Hkv, dk, dv, qt, kvt)
    scale = 1.0 / math.sqrt(dk)
    for causal, softcap in ((False, 0.0), (True, 30.0)):
        o = torch.empty((B, Sq, Hq, dv), device="cuda", dtype=torch.float32)
        lse = torch.empty((B, Hq, Sq), device="cuda", dtype=torch.float32)
        binding.attn_prefill_fwd_ex(to_dev(q), to_dev(k), to_dev(v), o, lse, scale=scale, causal=causal,
                                    softcap=softcap)
        torch.cuda.synchronize()
        ro, rl = oracle.prefill(q, k, v, scale, causal=causal, softcap=softcap)
        check_close(host(o), ro, "f32", "prefill %s/%s" % (qt, kvt))
        fin = np.isfinite(rl)
        assert np.abs(host(lse)[fin] - rl[fin]).max() < LSE_TOL


def test_prefill_f16_with_mask_sinks_bf16_out():
    B, Sq, Sk, Hq, Hkv, d = 2, 100, 260, 8, 2, 128
    q, k, v = prefill_case(410, B, Sq, Sk, Hq, Hkv, d, d, "f32", "f16")
    mask = synth.mask_case(410, 1, 1, Sq, Sk, kind="distance")
    sinks = np.random.Generator(np.random.PCG64(410)).standard_normal(Hq).astype(np.float32)
    o = torch.empty((B, Sq, Hq, d), device="cuda", dtype=torch.bfloat16)
    binding.attn_prefill_fwd_ex(to_dev(q), to_dev(k), to_dev(v), o, scale=d ** -0.5, sinks=dev(sinks),
                                mask=dev(mask), max_bias=8.0)
    torch.cuda.synchronize()
    ro, _ = oracle.prefill(q, k, v, d ** -0.5, sinks=sinks, mask=mask, max_bias=8.0)
    check_close(host(o), ro, "bf16", "fp16 K/V, fp32 Q, ALiBi mask, sinks")


@pytest.mark.parametrize("qt,kvt", [("f32", "f16"), ("f16", "f16"), ("f32", "bf16")])
def test_paged_operand_types(qt, kvt):
    print("paged q=%s kv=%s" % (qt, kvt), flush=True)
    B, Hq, Hkv, d, bs, Sq = 3, 16, 4, 128, 32, 2
    rng = np.random.Generator(np.random.PCG64(420))
    lens = rng.integers(100, 700, size=B, endpoint=True).astype(np.int32)
    nblk = (lens + bs - 1) // bs
    N = int(nblk.sum())
    max_blocks = int(nblk.max())
    perm = rng.permutation(N).astype(np.int32)
    table = np.zeros((B, max_blocks), dtype=np.int32)
    pos = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[pos:pos + nblk[b]]
        pos += nblk[b]
    q = synth.normal_typed(421, 0, (B, Sq, Hq, d), qt)
    kc = synth.normal_typed(421, 1, (N, Hkv, bs, d), kvt)
    vc = synth.normal_typed(421, 2, (N, Hkv, bs, d), kvt)
    o = torch.empty((B, Sq, Hq, d), device="cuda", dtype=torch.float32)
    Sk_max = int(lens.max())
    ws = torch.empty(binding.attn_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk_max, d, d), device="cuda",
                     dtype=torch.uint8)
    binding.attn_decode_fwd(to_dev(q), to_dev(kc), to_dev(vc), o, ws, scale=d ** -0.5, Sk_max=Sk_max, causal=True,
                            block_table=dev(table), seq_lens=dev(lens))
    torch.cuda.synchronize()
    ro, _ = oracle.decode_paged(q, kc, vc, table, lens, d ** -0.5, causal=True)
    check_close(host(o), ro, "f32", "paged %s/%s" % (qt, kvt))


@pytest.mark.parametrize("qt,kvt", [("f32", "f16"), ("f16", "f16"), ("f32", "bf16"), ("f16", "bf16")])
@pytest.mark.parametrize("cur", [False, True])
def test_gathered_operand_types(qt, kvt, cur):
    """Queries already in the rows' type are staged through LDS like the rows; the others are
    converted on load, one 16-byte piece per lane. With and without the token's own row (one
    more key of the last range) in the same types."""
    print("gathered q=%s rows=%s cur=%d" % (qt, kvt, cur), flush=True)
    T, Hq, n_rows, n_sel = 4, 128, 4096, 700
    case = synth.gathered_case(430, T, Hq, 576, 512, n_rows, n_sel, row_dim=576, future_keys=32)
    kv = synth.normal_typed(430, 1, (n_rows, 576), kvt)
    q = synth.normal_typed(430, 0, (T, Hq, 576), qt)
    kc = synth.normal_typed(430, 2, (T, 576), kvt) if cur else None
    kvd = to_dev(kv)
    kcd = to_dev(kc) if cur else None
    o = torch.empty((T, 1, Hq, 512), device="cuda", dtype=torch.float32)
    ws = torch.empty(binding.attn_decode_workspace_bytes(T, Hq, 1, 1, n_sel, 576, 512), device="cuda",
                     dtype=torch.uint8)
    binding.attn_decode_fwd(to_dev(q).view(T, 1, Hq, 576), kvd[:, :576], kvd[:, :512], o, ws, scale=1 / 24,
                            Sk_max=n_sel, causal=True, row_index=dev(case["row_index"]),
                            key_pos=dev(case["key_pos"]), q_pos=dev(case["q_pos"]),
                            k_cur=kcd, v_cur=None if kcd is None else kcd[:, :512])
    torch.cuda.synchronize()
    ro, _ = oracle.decode_gathered(q, kv, kv[:, :512], case["row_index"], case["key_pos"], case["q_pos"], 1 / 24,
                                   k_cur=kc, v_cur=None if kc is None else kc[:, :512])
    check_close(host(o[:, 0]), ro, "f32", "gathered %s rows, %s q, cur %d" % (kvt, qt, cur))
