"""Seeded random sweeps over the three attention entry points, each case against the fp64
oracle through the C ABI: head dims of the supported table, GQA ratios, ragged and
degenerate lengths (one query, one key, more queries than keys), and every option
combination. The fixed cases in the other files pin specific shapes; these cover the
space between them. Each case prints its parameters before it runs."""

import numpy as np
import pytest

from test_gpu_decode import check_gathered, check_paged
from test_gpu_prefill import check_case

pytestmark = pytest.mark.gpu

DIMS = [(16, 16), (32, 32), (64, 64), (96, 96), (128, 128), (192, 192), (256, 256), (192, 128)]


def _pick(rng, seq):
    return seq[int(rng.integers(len(seq)))]


@pytest.mark.parametrize("n", range(24))
def test_prefill_sweep(n):
    rng = np.random.default_rng([7001, n])
    dk, dv = _pick(rng, DIMS)
    Hkv = int(rng.integers(1, 4))
    Hq = Hkv * _pick(rng, [1, 2, 3, 4, 8])
    check_case(int(rng.integers(1, 3)), int(rng.integers(1, 300)), int(rng.integers(1, 300)), Hq, Hkv, dk, dv,
               causal=bool(rng.random() < 0.5), softcap=_pick(rng, [0.0, 0.0, float(rng.uniform(2, 60))]),
               sinks=bool(rng.random() < 0.4), o_dtype=_pick(rng, ["f32", "bf16"]),
               std=_pick(rng, [0.5, 1.0, 2.0]), seed=7100 + n)


@pytest.mark.parametrize("n", range(12))
def test_paged_sweep(n):
    rng = np.random.default_rng([7002, n])
    dk, dv = _pick(rng, DIMS)
    Hkv = int(rng.integers(1, 5))
    hi = int(rng.integers(4, 2600))
    check_paged(int(rng.integers(1, 6)), Hkv * _pick(rng, [1, 2, 4, 8, 16]), Hkv, dk, dv,
                int(rng.integers(1, hi + 1)), hi, bs=_pick(rng, [16, 32, 64, 128]), Sq=int(rng.integers(1, 5)),
                causal=bool(rng.random() < 0.5), softcap=_pick(rng, [0.0, float(rng.uniform(2, 60))]),
                sinks=bool(rng.random() < 0.4), o_dtype=_pick(rng, ["f32", "bf16"]), seed=7200 + n)


@pytest.mark.parametrize("n", range(8))
def test_gathered_sweep(n):
    rng = np.random.default_rng([7003, n])
    n_sel = int(rng.integers(1, 1500))
    check_gathered(int(rng.integers(1, 5)), _pick(rng, [16, 20, 64, 128]), 4096, n_sel,
                   causal=bool(rng.random() < 0.7), softcap=_pick(rng, [0.0, float(rng.uniform(5, 60))]),
                   sinks=bool(rng.random() < 0.4), o_dtype=_pick(rng, ["f32", "bf16"]),
                   future=_pick(rng, [0, min(32, n_sel)]), v_offset=_pick(rng, [0, 64]), seed=7300 + n,
                   shuffle=bool(rng.random() < 0.3), with_cur=bool(rng.random() < 0.5))
