"""GPU parity of attn_decode_fwd (paged mode) against the fp64 CPU oracle (through the C ABI)."""

import math

import numpy as np
import pytest
import torch

import oracle
from attention_flash_attn_amd import binding, synth
from gpu_util import check_close, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def run_paged(case, scale, causal, softcap, o_dtype, Sk_max):
    q = dev_bf16(case["q"])
    kc, vc = dev_bf16(case["k_cache"]), dev_bf16(case["v_cache"])
    table = dev(case["block_table"])
    lens = dev(case["seq_lens"])
    B, Sq, Hq, dk = q.shape
    Hkv = kc.shape[1]
    dv = vc.shape[3]
    o = torch.empty((B, Sq, Hq, dv), device="cuda", dtype=torch.float32 if o_dtype == "f32" else torch.bfloat16)
    nbytes = binding.attn_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk_max, dk, dv)
    ws = torch.empty(nbytes, device="cuda", dtype=torch.uint8)
    sinks = dev(case["sinks"]) if case["sinks"] is not None else None
    binding.attn_decode_fwd(q, kc, vc, o, ws, scale=scale, Sk_max=Sk_max, causal=causal, softcap=softcap,
                            sinks=sinks, block_table=table, seq_lens=lens)
    torch.cuda.synchronize()
    return o


def check_paged(B, Hq, Hkv, dk, dv, lo, hi, bs=64, Sq=1, causal=False, softcap=0.0, sinks=False, o_dtype="f32",
                seed=200, lens=None):
    print("paged B=%d Hq=%d Hkv=%d dk=%d dv=%d len[%d,%d] bs=%d Sq=%d causal=%d softcap=%g sinks=%d %s" %
          (B, Hq, Hkv, dk, dv, lo, hi, bs, Sq, causal, softcap, sinks, o_dtype), flush=True)
    case = synth.paged_case(seed, B, Hq, Hkv, dk, dv, lo, hi, block_size=bs, Sq=Sq, sinks=sinks, lens=lens)
    scale = 1.0 / math.sqrt(dk)
    Sk_max = int(hi)
    o = run_paged(case, scale, causal, softcap, o_dtype, Sk_max)
    ro, _ = oracle.decode_paged(case["q"], case["k_cache"], case["v_cache"], case["block_table"], case["seq_lens"],
                                scale, causal=causal, softcap=softcap, sinks=case["sinks"])
    return check_close(host(o), ro, o_dtype, "paged decode")


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 32), (64, 64), (96, 96), (128, 128), (192, 192), (256, 256),
                                   (192, 128)])
def test_paged_head_dims(dk, dv):
    check_paged(3, 8, 2, dk, dv, 1, 1300, o_dtype="f32")


@pytest.mark.parametrize("bs", [16, 32, 64, 128])
def test_paged_block_sizes(bs):
    check_paged(4, 16, 2, 128, 128, 30, 2100, bs=bs, o_dtype="bf16", seed=201)


def test_paged_gqa_ratios_and_features():
    check_paged(5, 32, 1, 64, 64, 500, 1500, o_dtype="f32", seed=202)                 # 32 query heads, 1 KV head
    check_paged(3, 4, 4, 128, 128, 1, 700, o_dtype="f32", softcap=3.0, sinks=True, seed=203)
    check_paged(2, 16, 8, 128, 128, 600, 600, Sq=4, causal=True, o_dtype="f32", seed=204)   # Sq > 1 causal
    check_paged(2, 8, 1, 128, 128, 0, 5, o_dtype="f32", seed=205, lens=[0, 5])        # empty sequence


def test_paged_causal_more_queries_than_keys():
    """Causal decode with Sq > L_b: query i sits at L_b - Sq + i, so the first Sq - L_b rows
    see no key and are 0 (the prefill's bottom-right alignment and empty-row rule)."""
    check_paged(3, 16, 2, 128, 128, 2, 40, Sq=6, causal=True, o_dtype="f32", seed=207, lens=[2, 6, 40])


def test_paged_block_permutation_invariance():
    case = synth.paged_case(206, 3, 8, 1, 128, 128, 100, 1000)
    o1 = run_paged(case, 0.09, False, 0.0, "f32", 1000)
    # move every block to a new physical slot and rewrite the table
    N = case["k_cache"].shape[0]
    perm = np.random.default_rng(5).permutation(N)
    case2 = dict(case)
    case2["k_cache"] = np.empty_like(case["k_cache"])
    case2["v_cache"] = np.empty_like(case["v_cache"])
    case2["k_cache"][perm] = case["k_cache"]
    case2["v_cache"][perm] = case["v_cache"]
    t = case["block_table"].copy()
    nblk = (case["seq_lens"] + 63) // 64
    for b in range(3):
        t[b, :nblk[b]] = perm[t[b, :nblk[b]]]
    case2["block_table"] = t
    o2 = run_paged(case2, 0.09, False, 0.0, "f32", 1000)
    assert torch.equal(o1, o2)


def test_config4_full_size():
    """Every output element of the paged decode workload (64 sequences of up to 32768 keys)."""
    c = synth.CONFIGS["c4_paged_gqa_decode"]
    print("full-size c4 paged decode, every element", flush=True)
    case = synth.paged_case(c["seed"], c["B"], c["Hq"], c["Hkv"], c["dk"], c["dv"], c["len_lo"], c["len_hi"],
                            block_size=c["block_size"])
    o = run_paged(case, c["scale"], False, 0.0, "bf16", c["len_hi"])
    ro, _ = oracle.decode_paged(case["q"], case["k_cache"], case["v_cache"], case["block_table"],
                                case["seq_lens"], c["scale"])
    err, cos = check_close(host(o), ro, "bf16", "config 4")
    print("config 4, %d elements: max err %.3g cos %.8f" % (ro.size, err, cos))


def _planned_splits(B, Hq, Hkv, Sq, Sk_max, dk, dv):
    """Number of key splits the library plans, read back from the workspace size
    (rows * n_split * (dv + 2) fp32, rounded up to 256 bytes)."""
    ws = binding.attn_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk_max, dk, dv)
    rows = B * Sq * Hq
    n_split = ws // (rows * (dv + 2) * 4)
    assert ws - n_split * rows * (dv + 2) * 4 < 256, "workspace of %d bytes is not a whole number of splits" % ws
    return n_split


def test_paged_split_lengths_512_1024():
    """Shapes whose (sequence, KV head) count plans 512- and 1024-key splits."""
    assert _planned_splits(8, 16, 8, 1, 20000, 128, 128) == -(-20000 // 512)
    check_paged(8, 16, 8, 128, 128, 9000, 20000, seed=210)
    assert _planned_splits(16, 8, 8, 1, 20000, 64, 64) == -(-20000 // 1024)
    check_paged(16, 8, 8, 64, 64, 12000, 20000, causal=True, Sq=1, o_dtype="bf16", seed=211)
    assert _planned_splits(16, 64, 8, 2, 20000, 64, 64) == -(-20000 // 1024)      # 16 columns per KV head
    check_paged(16, 64, 8, 64, 64, 15000, 20000, Sq=2, causal=True, seed=212)


def test_paged_split_length_3072():
    """A split length that is a multiple of 1024 but not a power of two (3072 keys: 7
    splits of 20000 keys for 48 sequences x 8 KV heads), sequences ending inside, at and
    just past a split boundary."""
    assert _planned_splits(48, 16, 8, 1, 20000, 128, 128) == -(-20000 // 3072)
    lens = np.array([3072, 3073, 6144, 6143, 20000, 1, 9215, 9216, 12289, 17000, 33, 3071] * 4, np.int32)
    check_paged(48, 16, 8, 128, 128, 1, 20000, seed=213, lens=lens)


def test_paged_draft_tokens_3072_key_splits():
    """4 causal draft tokens x 8 heads per KV head (the 32-column instance) at 3072-key splits,
    every output compared: sequences ending inside, at and just past split boundaries, shorter
    than the draft, and a single key."""
    assert _planned_splits(48, 64, 8, 4, 20000, 128, 128) == -(-20000 // 3072)
    lens = np.array([3072, 3075, 6144, 6146, 20000, 1, 9215, 9216, 12289, 17000, 33, 3071] * 4, np.int32)
    check_paged(48, 64, 8, 128, 128, 1, 20000, Sq=4, causal=True, o_dtype="bf16", seed=214, lens=lens)


def test_config4_shape_draft_tokens_6144_key_splits():
    """The workload's shape with 4 causal draft tokens per sequence: 32 query columns per KV
    head take the 32-column instance and 6144-key splits. Sequences of the longest,
    shortest and a few other lengths are compared with the oracle."""
    c = synth.CONFIGS["c4_paged_gqa_decode"]
    assert _planned_splits(c["B"], c["Hq"], c["Hkv"], 4, c["len_hi"], c["dk"], c["dv"]) == -(-c["len_hi"] // 6144)
    print("config 4 shape, 4 draft tokens, causal", flush=True)
    case = synth.paged_case(c["seed"], c["B"], c["Hq"], c["Hkv"], c["dk"], c["dv"], c["len_lo"], c["len_hi"],
                            block_size=c["block_size"], Sq=4)
    o = run_paged(case, c["scale"], True, 0.0, "bf16", c["len_hi"])
    batches = [0, 1, int(np.argmax(case["seq_lens"])), int(np.argmin(case["seq_lens"])), 40, 63]
    ro, _ = oracle.decode_paged(case["q"], case["k_cache"], case["v_cache"], case["block_table"],
                                case["seq_lens"], c["scale"], causal=True, batches=batches)
    err, cos = check_close(host(o)[batches], ro, "bf16", "config 4 shape, 4 draft tokens")
    print("4 draft tokens: max err %.3g cos %.8f" % (err, cos))


# ---------------------------------------------------------------- gathered rows (MLA-style)
def run_gathered(case, Hq, dk, dv, scale, causal=True, softcap=0.0, sinks=None, o_dtype="bf16", v_offset=0,
                 cur=None):
    kv = dev_bf16(case["kv"])
    q = dev_bf16(case["q"]).view(case["q"].shape[0], 1, Hq, dk)
    T, n_sel = case["row_index"].shape
    o = torch.empty((T, 1, Hq, dv), device="cuda", dtype=torch.float32 if o_dtype == "f32" else torch.bfloat16)
    nbytes = binding.attn_decode_workspace_bytes(T, Hq, 1, 1, n_sel, dk, dv)
    ws = torch.empty(nbytes, device="cuda", dtype=torch.uint8)
    k_rows = kv[:, :dk] if v_offset == 0 else kv[:, :dk]
    v_rows = kv[:, v_offset:v_offset + dv]
    k_cur = v_cur = None
    if cur is not None:
        cd = dev_bf16(cur)
        k_cur, v_cur = cd[:, :dk], cd[:, v_offset:v_offset + dv]
    binding.attn_decode_fwd(q, k_rows, v_rows, o, ws, scale=scale, Sk_max=n_sel, causal=causal, softcap=softcap,
                            sinks=None if sinks is None else dev(sinks), row_index=dev(case["row_index"]),
                            key_pos=dev(case["key_pos"]), q_pos=dev(case["q_pos"]), dk=dk, dv=dv,
                            k_cur=k_cur, v_cur=v_cur)
    torch.cuda.synchronize()
    return o[:, 0]


def check_gathered(T, Hq, n_rows, n_sel, causal=True, softcap=0.0, sinks=False, o_dtype="f32", future=0,
                   v_offset=0, seed=300, shuffle=False, with_cur=False):
    dk, dv = 576, 512
    print("gathered T=%d Hq=%d rows=%d n_sel=%d causal=%d softcap=%g sinks=%d %s future=%d v_offset=%d cur=%d" %
          (T, Hq, n_rows, n_sel, causal, softcap, sinks, o_dtype, future, v_offset, with_cur), flush=True)
    case = synth.gathered_case(seed, T, Hq, dk, dv, n_rows, n_sel, row_dim=576, sinks=sinks, future_keys=future)
    if shuffle:
        perm = np.random.default_rng(seed).permutation(n_sel)
        case["row_index"] = np.ascontiguousarray(case["row_index"][:, perm])
        case["key_pos"] = np.ascontiguousarray(case["key_pos"][:, perm])
    scale = 1.0 / math.sqrt(dk)
    cur = synth.normal_bf16(seed, 9, (T, 576)) if with_cur else None
    o = run_gathered(case, Hq, dk, dv, scale, causal, softcap, case["sinks"], o_dtype, v_offset, cur)
    kv = case["kv"]
    ro, _ = oracle.decode_gathered(case["q"], kv[:, :dk], kv[:, v_offset:v_offset + dv], case["row_index"],
                                   case["key_pos"], case["q_pos"], scale, causal=causal, softcap=softcap,
                                   sinks=case["sinks"], k_cur=None if cur is None else cur[:, :dk],
                                   v_cur=None if cur is None else cur[:, v_offset:v_offset + dv])
    check_close(host(o), ro, o_dtype, "gathered decode")
    return host(o), ro


def test_gathered_small_and_ragged():
    check_gathered(3, 64, 4096, 300)                                  # ragged last split
    check_gathered(2, 20, 2048, 65, o_dtype="bf16", seed=301)         # heads not a multiple of 16
    check_gathered(2, 128, 4096, 1, seed=302)                         # a single selected row


def test_gathered_position_mask():
    check_gathered(4, 32, 8192, 512, future=64, seed=303)             # 64 keys per token lie after it
    check_gathered(2, 32, 8192, 512, causal=False, future=64, seed=304)
    # keys after the token scattered over every range and step (a step with all keys live skips
    # the mask, one with any key after the token takes it)
    check_gathered(3, 64, 8192, 700, future=200, shuffle=True, seed=308)
    check_gathered(2, 128, 8192, 2048, future=77, shuffle=True, o_dtype="bf16", seed=309)


def test_gathered_softcap_sinks_order_and_layout():
    check_gathered(2, 64, 4096, 700, softcap=30.0, sinks=True, seed=305)
    check_gathered(2, 64, 4096, 700, shuffle=True, seed=306)          # selection order does not matter
    # value stored after a 64-wide field ([k_pe | latent] rows): v = row[64:576], k = row[0:576]
    case_rows = 4096
    check_gathered(2, 32, case_rows, 333, v_offset=64, seed=307)


def test_config5_full_size():
    c = synth.CONFIGS["c5_gathered_mla_decode"]
    print("full-size c5 gathered decode", flush=True)
    o, ro = check_gathered(c["T"], c["Hq"], c["n_rows"], c["n_sel"], o_dtype="bf16", seed=c["seed"])
    print("config 5: max err %.3g" % np.abs(o - ro).max())


def test_gathered_bitwise_repeatable():
    """Two launches of the gathered decode on the same inputs give identical bits (the
    split partials are merged in a fixed order)."""
    c = synth.CONFIGS["c5_gathered_mla_decode"]
    print("gathered decode repeatability at the workload shape", flush=True)
    case = synth.gathered_case(c["seed"], c["T"], c["Hq"], c["dk"], c["dv"], c["n_rows"], c["n_sel"],
                               row_dim=c["row_dim"], future_keys=64)
    outs = [run_gathered(case, c["Hq"], c["dk"], c["dv"], c["scale"], o_dtype=od) for od in ("bf16", "bf16", "f32",
                                                                                          "f32")]
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(outs[2].view(torch.int32), outs[3].view(torch.int32))


def test_gathered_current_row():
    """The token's own row joins the selected rows as key n_prior (always live)."""
    check_gathered(5, 128, 4096, 100, with_cur=True, seed=320)                    # one ragged split + 1
    check_gathered(3, 64, 4096, 256, with_cur=True, seed=321)                     # 257 keys: one extra step
    check_gathered(4, 128, 8192, 2048, with_cur=True, future=64, o_dtype="bf16", seed=322)
    check_gathered(3, 128, 4096, 300, with_cur=True, v_offset=64, softcap=30.0, sinks=True, seed=323)


def test_gathered_long_selection():
    """4096 and more selected rows take 512-key splits, 16384 and more 1024-key splits; the
    last split can hold a full index table plus the current row."""
    check_gathered(2, 64, 16384, 4096, with_cur=True, seed=325)                   # 8 full splits + 1 row
    check_gathered(2, 32, 16384, 5000, future=64, o_dtype="bf16", seed=326)      # ragged tenth split
    check_gathered(1, 64, 16384, 4608, with_cur=True, v_offset=64, seed=327)     # separate value rows
    # 16384 and more take 1024-key splits: full index tables of 1024 rows (+ the current row)
    check_gathered(2, 32, 32768, 16384, with_cur=True, seed=330)
    check_gathered(1, 20, 32768, 17000, future=32, o_dtype="bf16", seed=331)


def test_gathered_separate_value_rows():
    """Value rows in an array of their own (same row stride as the key rows), with and
    without the token's own rows."""
    for T, Hq, n_sel, cur, seed in [(3, 64, 300, False, 328), (2, 128, 700, True, 329)]:
        print("gathered separate value rows T=%d Hq=%d n_sel=%d cur=%d" % (T, Hq, n_sel, cur), flush=True)
        case = synth.gathered_case(seed, T, Hq, 576, 512, 4096, n_sel, row_dim=576, future_keys=16)
        vrows = synth.normal_bf16(seed, 7, (4096, 576))
        kv, q = dev_bf16(case["kv"]), dev_bf16(case["q"]).view(T, 1, Hq, 576)
        vd = dev_bf16(vrows)
        o = torch.empty((T, 1, Hq, 512), device="cuda", dtype=torch.float32)
        ws = torch.empty(binding.attn_decode_workspace_bytes(T, Hq, 1, 1, n_sel, 576, 512), device="cuda",
                         dtype=torch.uint8)
        kcur = synth.normal_bf16(seed, 9, (T, 576)) if cur else None
        vcur = synth.normal_bf16(seed, 10, (T, 576)) if cur else None
        binding.attn_decode_fwd(q, kv, vd[:, :512], o, ws, scale=1 / 24, Sk_max=n_sel, causal=True,
                                row_index=dev(case["row_index"]), key_pos=dev(case["key_pos"]),
                                q_pos=dev(case["q_pos"]), dk=576, dv=512,
                                k_cur=None if kcur is None else dev_bf16(kcur),
                                v_cur=None if vcur is None else dev_bf16(vcur)[:, :512])
        torch.cuda.synchronize()
        ro, _ = oracle.decode_gathered(case["q"], case["kv"], vrows[:, :512], case["row_index"], case["key_pos"],
                                       case["q_pos"], 1 / 24, causal=True, k_cur=kcur,
                                       v_cur=None if vcur is None else vcur[:, :512])
        check_close(host(o[:, 0]), ro, "f32", "gathered decode, separate value rows")


def test_gathered_only_current_row_live():
    """Every selected key lies after the token: the output is the current row's value."""
    o, ro = check_gathered(3, 64, 2048, 96, with_cur=True, future=96, seed=324)
    cur = synth.bf16_bits_to_f32(synth.normal_bf16(324, 9, (3, 576)))
    np.testing.assert_allclose(ro, np.broadcast_to(cur[:, None, :512], ro.shape), rtol=0, atol=1e-12)


def test_paged_column_groups_small_dims():
    """32-column groups (the instance that addresses K/V as block base + in-block offset) at value
    widths whose 16-row halves fill no, one and three whole 1 KB segments (dv = 16, 32, 96), with
    16-key blocks so every step spans two blocks, and lengths down to one key."""
    check_paged(2, 16, 2, 16, 16, 30, 300, bs=16, Sq=4, causal=True, seed=333)
    check_paged(2, 32, 4, 32, 32, 17, 250, bs=16, Sq=3, causal=True, softcap=20.0, seed=334)
    check_paged(3, 24, 3, 96, 96, 1, 333, bs=128, Sq=4, sinks=True, o_dtype="bf16", seed=335)
    check_paged(2, 16, 2, 96, 96, 1, 40, bs=16, Sq=4, causal=True, seed=336, lens=[1, 40])


def test_paged_many_query_columns():
    """Sq * Hq / Hkv > 32 query columns per KV head (several draft tokens): column groups of 32."""
    check_paged(3, 64, 8, 128, 128, 200, 700, Sq=8, causal=True, seed=330)         # 64 columns
    check_paged(2, 32, 2, 64, 64, 100, 400, Sq=5, causal=True, o_dtype="bf16", seed=331)  # 80 columns
    check_paged(2, 16, 1, 256, 256, 150, 300, Sq=3, causal=False, softcap=10.0, sinks=True, seed=332)
