"""Seeded input generators: bf16 rounding, determinism and index structure."""

import numpy as np
import torch

from attention_flash_attn_amd import synth


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.Generator(np.random.PCG64(0))
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.0e38, 65504.0], np.float32)])
    ours = synth.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(synth.to_bf16_bits(back), ours)


def test_prefill_case_deterministic_and_shaped():
    a = synth.prefill_case(7, 1, 5, 6, 4, 2, 16, 8, std=0.5, sinks=True)
    b = synth.prefill_case(7, 1, 5, 6, 4, 2, 16, 8, std=0.5, sinks=True)
    for key in ("q", "k", "v", "sinks"):
        assert np.array_equal(a[key], b[key])
    assert a["q"].shape == (1, 5, 4, 16) and a["k"].shape == (1, 6, 2, 16) and a["v"].shape == (1, 6, 2, 8)
    assert a["q"].dtype == np.uint16 and a["sinks"].dtype == np.float32
    std = synth.bf16_bits_to_f32(synth.prefill_case(8, 1, 256, 256, 8, 8, 64, 64, std=0.5)["q"]).std()
    assert abs(std - 0.5) < 0.01


def test_paged_case_block_table_is_a_permutation():
    c = synth.paged_case(3, B=5, Hq=4, Hkv=2, dk=8, dv=8, len_lo=1, len_hi=300, block_size=64)
    lens, table = c["seq_lens"], c["block_table"]
    nblk = (lens + 63) // 64
    used = np.concatenate([table[b, :nblk[b]] for b in range(5)])
    assert np.array_equal(np.sort(used), np.arange(int(nblk.sum())))
    assert c["k_cache"].shape[0] == int(nblk.sum())
    assert (lens >= 1).all() and (lens <= 300).all()


def test_gathered_case_selection():
    c = synth.gathered_case(5, T=4, Hq=2, dk=16, dv=8, n_rows=1024, n_sel=64, future_keys=4)
    ri, kp, qp = c["row_index"], c["key_pos"], c["q_pos"]
    assert ri.shape == (4, 64) and kp.dtype == np.float32
    for t in range(4):
        assert len(set(ri[t].tolist())) == 64
        assert (kp[t, :60] <= qp[t]).all() and (kp[t, 60:] > qp[t]).all()
    assert ri.min() >= 0 and ri.max() < 1024
