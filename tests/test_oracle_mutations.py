"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pin set catches every one of them. This shows the pins constrain each part
of the definition: the scale, the softcap, the sink term, the causal alignment,
the GQA head map, the value operand, the lse, the paged and gathered indexing,
the draft rows' causal offset in paged decode and the widening of bf16 bit patterns."""

import importlib.util
import os
import sys
import types

import pytest

from oracle_pins import PINS

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.py")

MUTATIONS = {
    "dropped_scale": ("x = (qrows @ keys.T) * scale", "x = (qrows @ keys.T)"),
    "softcap_without_division": ("np.tanh(x / softcap)", "np.tanh(x)"),
    "sink_sign": ("np.exp(float(sink) - m_safe)", "np.exp(m_safe - float(sink))"),
    "sink_left_out": ("Z = Z + np.exp(float(sink) - m_safe)", "Z = Z"),
    "causal_top_left": ("live = _causal_live(rows + (Sk - Sq), Sk)", "live = _causal_live(rows, Sk)"),
    "causal_strict": ("return j[None, :] <= np.asarray(q_positions)[:, None]",
                      "return j[None, :] < np.asarray(q_positions)[:, None]"),
    "gqa_modulo": ("g = h // group\n            sink", "g = h % Hkv\n            sink"),
    "keys_as_values": ("num = e @ values", "num = e @ keys[:, :dv]"),
    "lse_without_log": ("m_safe + np.log(np.where(Z > 0, Z, 1.0))", "m_safe + np.where(Z > 0, Z, 1.0)"),
    "empty_row_not_zero": ("o[ok] = num[ok] / Z[ok, None]", "o[:] = num / np.where(Z > 0, Z, 1.0)[:, None] + (~ok)[:, None]"),
    "paged_slot_index": ("slot = j % bs", "slot = (j + 1) % bs"),
    "paged_block_index": ("phys = block_table[b, j // bs]", "phys = block_table[b, j % block_table.shape[1]]"),
    "gathered_strict_position": ("(key_pos[t] <= float(q_pos[t]))", "(key_pos[t] < float(q_pos[t]))"),
    "gathered_value_rows": ("V = _as_f64(v_rows[r])", "V = _as_f64(v_rows[np.sort(r)])"),
    "max_ignores_mask": ("x = np.where(live, x, -np.inf)", "x = np.where(live, x, -1e3)"),
    "mask_before_softcap": ("    if softcap != 0.0:\n        x = softcap * np.tanh(x / softcap)\n    if live is None:",
                            "    if bias is not None:\n        x = x + np.where(np.asarray(bias) > -np.inf, bias, 0.0)\n"
                            "    if softcap != 0.0:\n        x = softcap * np.tanh(x / softcap)\n    if live is None:"),
    "mask_sign": ("x = x + np.where(live, bias, 0.0)", "x = x - np.where(live, bias, 0.0)"),
    "mask_head_by_kv_group": ("mask[b % mask.shape[0], h % mask.shape[1]]", "mask[b % mask.shape[0], g % mask.shape[1]]"),
    "alibi_exponent_off_by_one": ("m0 ** (h + 1)", "m0 ** h"),
    "alibi_m1_base": ("m1 = 2.0 ** (-max_bias / 2.0 / n_log2)", "m1 = 2.0 ** (-max_bias / n_log2)"),
    "alibi_slope_ignored": ("bias = slopes[h] * mrows", "bias = mrows"),
    "q4_0_nibble_order": ("q = np.concatenate([nib & 0x0F, nib >> 4], axis=1)", "q = np.stack([nib & 0x0F, nib >> 4], axis=2).reshape(len(nib), 32)"),
    "q4_0_no_offset": (".astype(np.float64) - 8.0", ".astype(np.float64)"),
    "q8_0_unsigned": ("q = blk[:, 2:].view(np.int8)", "q = blk[:, 2:].view(np.uint8)"),
    "current_row_masked": ("live_row = np.concatenate([live_row, [True]])",
                           "live_row = np.concatenate([live_row, [False]])"),
    "current_row_wrong_token": ("_as_f64(np.asarray(k_cur)[t])[None, :]", "_as_f64(np.asarray(k_cur)[0])[None, :]"),
    "tail_absorb_layout_r_major": ("u[:, h, :] = o[:, h, :] @ wa[h].T", "u[:, h, :] = o[:, h, :] @ wa[h].reshape(R, DV)"),
    "tail_absorb_wrong_head": ("u[:, h, :] = o[:, h, :] @ wa[h].T", "u[:, h, :] = o[:, h, :] @ wa[(h + 1) % H].T"),
    "tail_concat_value_major": ("y = u.reshape(T, H * DV) @ wo", "y = u.transpose(0, 2, 1).reshape(T, H * DV) @ wo"),
    "bf16_widen_shift_15": ("(b.astype(np.uint32) << 16)", "(b.astype(np.uint32) << 15)"),
    "paged_draft_offset_plus_one": ("np.arange(Sq) + (L - Sq)", "np.arange(Sq) + (L - Sq + 1)"),
    "paged_draft_all_at_last_key": ("np.arange(Sq) + (L - Sq)", "np.full(Sq, L - 1)"),
}


def _mutant(old, new):
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: %r" % old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pname, pin in PINS.items():
        try:
            pin(mod)
        except AssertionError:
            caught.append(pname)
        except Exception:  # a crash also exposes the mistake
            caught.append(pname + "(error)")
    assert caught, "no pin caught the planted mistake %s" % name
