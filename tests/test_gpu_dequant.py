"""GPU parity of attn_dequant_fp16 (the quantized-KV pre-pass) against the oracle: bit-exact
fp16 (byte work: the kernel and the oracle round the exact product d * q once), and an
end-to-end paged decode over dequantized K/V."""

import math

import numpy as np
import pytest
import torch

import oracle
from attention_flash_attn_amd import binding
from gpu_util import check_close, dev, host

pytestmark = pytest.mark.gpu


def random_blocks(seed, n, fmt):
    rng = np.random.Generator(np.random.PCG64(seed))
    size = {"q8_0": 34, "q4_0": 18}[fmt]
    raw = rng.integers(0, 256, size=(n, size), dtype=np.uint8)
    d = (rng.standard_normal(n) * 0.05).astype(np.float16)     # signed scales
    raw[:, :2] = d.view(np.uint8).reshape(n, 2)
    return raw.reshape(-1)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("n", [1, 255, 256, 257, 4099])
def test_dequant_bit_exact(fmt, n):
    print("dequant %s n_blocks=%d" % (fmt, n), flush=True)
    raw = random_blocks(500 + n, n, fmt)
    out = torch.empty(n * 32, device="cuda", dtype=torch.float16)
    binding.attn_dequant_fp16(dev(raw), fmt, out)
    torch.cuda.synchronize()
    want = oracle.dequant_blocks(raw, fmt).astype(np.float16)
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_paged_decode_over_dequantized_cache():
    """q8_0 K/V expanded by the pre-pass, then fp16 paged decode, against the oracle on the
    block values."""
    B, Hq, Hkv, d, bs = 2, 8, 2, 128, 64
    lens = np.array([300, 1000], dtype=np.int32)
    nblk = (lens + bs - 1) // bs
    N = int(nblk.sum())
    table = np.zeros((B, int(nblk.max())), dtype=np.int32)
    table[0, :nblk[0]] = np.arange(nblk[0])
    table[1, :nblk[1]] = nblk[0] + np.arange(nblk[1])
    nvals = N * Hkv * bs * d
    kraw, vraw = random_blocks(510, nvals // 32, "q8_0"), random_blocks(511, nvals // 32, "q8_0")
    kc = torch.empty(nvals, device="cuda", dtype=torch.float16)
    vc = torch.empty(nvals, device="cuda", dtype=torch.float16)
    binding.attn_dequant_fp16(dev(kraw), "q8_0", kc)
    binding.attn_dequant_fp16(dev(vraw), "q8_0", vc)
    q = np.random.Generator(np.random.PCG64(512)).standard_normal((B, 1, Hq, d)).astype(np.float32)
    o = torch.empty((B, 1, Hq, d), device="cuda", dtype=torch.float32)
    ws = torch.empty(binding.attn_decode_workspace_bytes(B, Hq, Hkv, 1, int(lens.max()), d, d), device="cuda",
                     dtype=torch.uint8)
    binding.attn_decode_fwd(dev(q), kc.view(N, Hkv, bs, d), vc.view(N, Hkv, bs, d), o, ws, scale=d ** -0.5,
                            Sk_max=int(lens.max()), block_table=dev(table), seq_lens=dev(lens))
    torch.cuda.synchronize()
    kvals = oracle.dequant_blocks(kraw, "q8_0").astype(np.float16).reshape(N, Hkv, bs, d)
    vvals = oracle.dequant_blocks(vraw, "q8_0").astype(np.float16).reshape(N, Hkv, bs, d)
    ro, _ = oracle.decode_paged(q, kvals, vvals, table, lens, d ** -0.5)
    check_close(host(o), ro, "f32", "decode over dequantized q8_0 cache")
