"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments with the documented status before any HIP
call (so these run without a GPU; no compute call is made)."""

import ctypes
import os
import re

import pytest

import attention_flash_attn_amd as attn
from attention_flash_attn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.library_path()),
                                reason="libattn.so not built (run __graft_entry__.build())")

FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first


def declared_functions():
    with open(HEADER) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = binding.load_library()
    names = declared_functions()
    assert {"attn_prefill_fwd", "attn_prefill_fwd_ex", "attn_decode_fwd",
            "attn_decode_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), "symbol %s missing from libattn.so" % n


def test_abi_version_matches_header():
    with open(HEADER) as f:
        ver = int(re.search(r"#define ATTN_ABI_VERSION (\d+)", f.read()).group(1))
    assert attn.attn_abi_version() == ver
    assert attn.attn_status_string(0) == "ok"
    assert attn.attn_status_string(2) == "unsupported configuration"


def prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, od=0, lse=None, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, dk=64, dv=64,
             scale=0.125, causal=0, softcap=0.0, sinks=None, stream=None)
    a.update(kw)
    return lib.attn_prefill_fwd(a["q"], a["k"], a["v"], a["o"], a["od"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                a["Sq"], a["Sk"], a["dk"], a["dv"], a["scale"], a["causal"], a["softcap"],
                                a["sinks"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1),
    (dict(o=None), 1),
    (dict(B=0), 1),
    (dict(Sk=0), 1),
    (dict(Hq=3, Hkv=2), 1),
    (dict(scale=0.0), 1),
    (dict(scale=float("nan")), 1),
    (dict(softcap=-1.0), 1),
    (dict(od=7), 1),
    (dict(q=ctypes.c_void_p(0x10002)), 1),
    (dict(dk=48, dv=48), 2),
    (dict(dk=128, dv=64), 2),
    (dict(dk=576, dv=512), 2),
    (dict(B=65536, Hq=128, Sq=1024), 2),              # grid of more than 2^32 threads
])
def test_prefill_rejects(kw, status):
    lib = binding.load_library()
    assert prefill(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def prefill_ex(lib, **kw):
    a = dict(q=FAKE, qd=0, k=FAKE, v=FAKE, kvd=0, o=FAKE, od=0, lse=None, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, dk=64,
             dv=64, scale=0.125, causal=0, softcap=0.0, sinks=None, mask=FAKE, mb=1, mh=1, ms=8, max_bias=0.0,
             stream=None)
    a.update(kw)
    return lib.attn_prefill_fwd_ex(a["q"], a["qd"], a["k"], a["v"], a["kvd"], a["o"], a["od"], a["lse"], a["B"],
                                   a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["dk"], a["dv"], a["scale"], a["causal"],
                                   a["softcap"], a["sinks"], a["mask"], a["mb"], a["mh"], a["ms"], a["max_bias"],
                                   a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1),
    (dict(mb=0), 1),
    (dict(mh=0), 1),
    (dict(ms=6), 1),                                   # row stride below Sk
    (dict(ms=10), 1),                                  # not a multiple of 4
    (dict(mask=ctypes.c_void_p(0x10008)), 1),          # not 16-byte aligned
    (dict(max_bias=-1.0), 1),
    (dict(max_bias=float("inf")), 1),
    (dict(Sq=1 << 20, Sk=1 << 20, ms=1 << 20), 2),     # one mask slab of 2 TiB
    (dict(dk=48, dv=48), 2),
    (dict(qd=3), 1),                                   # unknown q dtype
    (dict(kvd=1), 1),                                  # fp32 K/V are not an operand type
])
def test_prefill_ex_rejects(kw, status):
    lib = binding.load_library()
    assert prefill_ex(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def decode(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, od=0, qd=0, kvd=0, B=2, Hq=8, Hkv=1, Sq=1, Sk_max=100, dk=128, dv=128,
             scale=0.1, causal=0, softcap=0.0, sinks=None, table=FAKE, bs=64, maxb=2, lens=FAKE,
             rows=None, kpos=None, qpos=None, n_sel=0, stride=0, kcur=None, vcur=None, ws=FAKE, ws_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return lib.attn_decode_fwd(a["q"], a["kc"], a["vc"], a["o"], a["od"], a["qd"], a["kvd"], a["B"], a["Hq"],
                               a["Hkv"], a["Sq"],
                               a["Sk_max"], a["dk"], a["dv"], a["scale"], a["causal"], a["softcap"], a["sinks"],
                               a["table"], a["bs"], a["maxb"], a["lens"], a["rows"], a["kpos"], a["qpos"],
                               a["n_sel"], a["stride"], a["kcur"], a["vcur"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1),
    (dict(table=None), 1),                                  # neither mode
    (dict(rows=FAKE, kpos=FAKE, qpos=FAKE, n_sel=100), 1),  # both modes
    (dict(lens=None), 1),
    (dict(bs=48), 1),
    (dict(maxb=1), 1),                                      # table too short for Sk_max
    (dict(ws_bytes=16), 1),
    (dict(ws=None), 1),
    (dict(Sq=1 << 12, Hq=512, Hkv=1), 2),                   # 2^21 query columns per KV head
    (dict(B=65536), 2),                                     # B is a grid dimension of at most 65535
    (dict(B=1024, Hq=1 << 16, Hkv=1 << 16), 2),             # 2^26 output rows for the combine
    (dict(table=None, rows=FAKE, kpos=FAKE, qpos=FAKE, n_sel=1 << 23, Sk_max=1 << 23, stride=576, dk=576,
          dv=512, B=256, Hq=128 * 2047), 2),                # 256 * 2047 head groups * 8192 ranges >= 2^31
    (dict(kcur=FAKE, vcur=FAKE), 1),                        # current rows in paged mode
    (dict(qd=5), 1),                                        # unknown q dtype
    (dict(kvd=1), 1),                                       # fp32 caches are not an operand type
    (dict(dk=100, dv=100), 2),
    (dict(table=None, rows=FAKE, kpos=FAKE, qpos=FAKE, n_sel=100, Hkv=2, Hq=8), 1),
    (dict(table=None, rows=FAKE, kpos=FAKE, qpos=FAKE, n_sel=100, stride=128), 2),          # gathered (128,128)
    (dict(table=None, rows=FAKE, kpos=FAKE, qpos=FAKE, n_sel=100, stride=576, dk=576, dv=512, Sq=2), 1),
    (dict(table=None, rows=FAKE, kpos=FAKE, qpos=FAKE, n_sel=99, stride=128), 1),
    (dict(table=None, rows=FAKE, kpos=None, qpos=FAKE, n_sel=100, stride=128), 1),
    (dict(table=None, rows=FAKE, kpos=FAKE, qpos=FAKE, n_sel=100, stride=576, dk=576, dv=512, Hq=128,
          kcur=FAKE), 1),                                   # k_cur without v_cur
    (dict(table=None, rows=FAKE, kpos=FAKE, qpos=FAKE, n_sel=100, stride=576, dk=576, dv=512, Hq=128,
          kcur=FAKE, vcur=ctypes.c_void_p(0x20000)), 1),    # v_cache == k_cache but v_cur != k_cur
])
def test_decode_rejects(kw, status):
    lib = binding.load_library()
    assert decode(lib, **kw) == status


def test_workspace_bytes():
    # paged, 64 sequences x 8 KV heads: 6144-key splits (6 splits of 32768 keys), so that
    # the expected non-empty splits fill one round of wave slots; (dv + 2) floats per row
    # per split
    n = attn.attn_decode_workspace_bytes(64, 64, 8, 1, 32768, 128, 128)
    assert n == (64 * 64 * 6 * 130 * 4 + 255) // 256 * 256
    # one sequence: 256-key splits keep about 4096 wavefronts busy
    n = attn.attn_decode_workspace_bytes(1, 8, 8, 1, 16384, 128, 128)
    assert n >= 1 * 8 * 64 * 130 * 4
    # gathered, 16 tokens x 128 heads (2 groups of 64) x 2048 keys: 8 ranges of 256 keys give
    # 256 workgroups; bf16 rows (dv * 2 bytes) plus fp32 (max, sum) per row per range
    n = attn.attn_decode_workspace_bytes(16, 128, 1, 1, 2048, 576, 512)
    assert n == (16 * 128 * 8 * (512 * 2 + 8) + 255) // 256 * 256
    assert attn.attn_decode_workspace_bytes(0, 64, 8, 1, 100, 128, 128) == 0
    # the longest key count an int holds: a whole number of splits, at most 65535 of them
    n = attn.attn_decode_workspace_bytes(1, 8, 8, 1, 2**31 - 1, 128, 128)
    row_split = 8 * 130 * 4
    assert 0 < n and (n // row_split) * row_split <= n < (n // row_split) * row_split + 256
    assert 1 <= n // row_split <= 65535
    assert attn.attn_decode_workspace_bytes(2, 6, 4, 1, 100, 128, 128) == 0
    # past the launch limits (2^26 output rows; B above 65535): no workspace size
    assert attn.attn_decode_workspace_bytes(1024, 1 << 16, 1 << 16, 1, 100, 128, 128) == 0
    assert attn.attn_decode_workspace_bytes(65536, 8, 8, 1, 100, 128, 128) == 0
    assert attn.attn_decode_workspace_bytes(1024, (1 << 16) - 64, 1, 1, 100, 128, 128) > 0


@pytest.mark.parametrize("fmt,src,dst,n,status", [
    (2, FAKE, FAKE, 4, 1),                                   # unknown format
    (0, FAKE, FAKE, -1, 1),
    (0, None, FAKE, 4, 1),
    (1, ctypes.c_void_p(0x10002), FAKE, 4, 1),                # misaligned source
    (0, FAKE, FAKE, 0, 0),                                    # nothing to do (no launch)
    (0, FAKE, FAKE, (1 << 30) - 63, 2),                       # four threads per block: grid past 2^32 threads
])
def test_dequant_rejects(fmt, src, dst, n, status):
    lib = binding.load_library()
    assert lib.attn_dequant_fp16(src, fmt, dst, n, None) == status


def tail(lib, **kw):
    a = dict(o=FAKE, wa=FAKE, wo=FAKE, y=FAKE, yd=0, T=16, H=8, R=128, DV=32, N=256, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.attn_mla_tail(a["o"], a["wa"], a["wo"], a["y"], a["yd"], a["T"], a["H"], a["R"], a["DV"], a["N"],
                             a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), 1),
    (dict(ws=None), 1),
    (dict(T=0), 1),
    (dict(yd=2), 1),                          # fp16 output is not offered
    (dict(R=96), 1),                          # latent width not a multiple of 128
    (dict(DV=24), 1),                         # v_head_dim not a multiple of 16
    (dict(H=3, DV=16), 1),                    # H * DV = 48, not a multiple of 128
    (dict(N=200), 1),                         # hidden width not a multiple of 128
    (dict(wo=ctypes.c_void_p(0x10008)), 1),   # misaligned weights
    (dict(wsb=1024), 1),                      # workspace too small
    (dict(T=1 << 27), 1),                     # T * N = 2^35 outputs: final-sum grid past 2^32 threads
])
def test_mla_tail_rejects(kw, status):
    lib = binding.load_library()
    assert tail(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def test_mla_tail_workspace_bytes():
    # u (bf16 [T, H*DV], rounded up to 256 bytes) + fp32 partials of every K slice
    n = attn.attn_mla_tail_workspace_bytes(16, 128, 512, 128, 7168)
    assert n >= 16 * 128 * 128 * 2 + 16 * 7168 * 4
    assert (n - 16 * 128 * 128 * 2) % (16 * 7168 * 4) == 0
    assert attn.attn_mla_tail_workspace_bytes(0, 128, 512, 128, 7168) == 0


# ---------------------------------------------------------------- binding shape checks
# The binding derives every size from q, k and v (or the caches) and checks each other
# tensor against them before any pointer is taken, so these run on CPU tensors: a shape
# mismatch raises INVALID_ARG naming the tensor (a correct shape only fails later, at the
# "must be on the GPU" check).
def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def _raises_shape(fn, name):
    with pytest.raises(binding.AttnError) as ei:
        fn()
    assert ei.value.status == binding.ATTN_ERR_INVALID_ARG
    assert name in str(ei.value) and "GPU" not in str(ei.value), str(ei.value)


def _prefill_args(**kw):
    import torch
    a = dict(q=_t(2, 8, 4, 64), k=_t(2, 8, 2, 64), v=_t(2, 8, 2, 64), o=_t(2, 8, 4, 64), lse=None, sinks=None)
    a.update(kw)
    return a


@pytest.mark.parametrize("name,bad", [
    ("o", dict(o=_t(2, 8, 4, 32))),
    ("o", dict(o=_t(1, 8, 4, 64))),
    ("k", dict(k=_t(2, 8, 2, 32))),
    ("k", dict(k=_t(1, 8, 2, 64))),
    ("v", dict(v=_t(2, 7, 2, 64))),
    ("lse", dict(lse=_t(2, 4, 9, dtype=None))),
    ("sinks", dict(sinks=_t(3))),
    ("q", dict(q=_t(2, 8, 64))),
])
def test_binding_prefill_rejects_mismatched_shapes(name, bad):
    a = _prefill_args(**bad)
    _raises_shape(lambda: binding.attn_prefill_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], scale=0.1,
                                                   sinks=a["sinks"]), name)
    _raises_shape(lambda: binding.attn_prefill_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], scale=0.1,
                                                      sinks=a["sinks"]), name)


def test_binding_prefill_good_shapes_reach_the_device_check():
    a = _prefill_args()
    with pytest.raises(binding.AttnError) as ei:
        binding.attn_prefill_fwd(a["q"], a["k"], a["v"], a["o"], None, scale=0.1)
    assert "GPU" in str(ei.value)


def _paged_args(**kw):
    import torch
    a = dict(q=_t(3, 1, 8, 64), kc=_t(10, 2, 16, 64), vc=_t(10, 2, 16, 64), o=_t(3, 1, 8, 64),
             table=_t(3, 4, dtype=torch.int32), lens=_t(3, dtype=torch.int32), sinks=None)
    a.update(kw)
    return a


@pytest.mark.parametrize("name,bad", [
    ("q's head dim", dict(q=_t(3, 1, 8, 32))),
    ("o", dict(o=_t(3, 1, 8, 32))),
    ("o", dict(o=_t(3, 2, 8, 64))),
    ("v_cache", dict(vc=_t(10, 1, 16, 64))),
    ("block_table", dict(table=_t(2, 4))),
    ("seq_lens", dict(lens=_t(4))),
    ("sinks", dict(sinks=_t(4))),
])
def test_binding_paged_rejects_mismatched_shapes(name, bad):
    a = _paged_args(**bad)
    _raises_shape(lambda: binding.attn_decode_fwd(a["q"], a["kc"], a["vc"], a["o"], _t(16), scale=0.1, Sk_max=64,
                                                  block_table=a["table"], seq_lens=a["lens"], sinks=a["sinks"]),
                  name)


def _gathered_args(**kw):
    import torch
    a = dict(q=_t(2, 1, 16, 576), rows=_t(100, 576), o=_t(2, 1, 16, 512), ri=_t(2, 5, dtype=torch.int32),
             kp=_t(2, 5, dtype=torch.float32), qp=_t(2, dtype=torch.int32))
    a.update(kw)
    return a


@pytest.mark.parametrize("name,bad", [
    ("o", dict(o=_t(2, 1, 16, 256))),
    ("key_pos", dict(kp=_t(2, 4))),
    ("q_pos", dict(qp=_t(3))),
    ("row_index", dict(ri=_t(2, 5, 1))),
    ("q's head dim", dict(q=_t(2, 1, 16, 512))),
])
def test_binding_gathered_rejects_mismatched_shapes(name, bad):
    a = _gathered_args(**bad)
    _raises_shape(lambda: binding.attn_decode_fwd(a["q"], a["rows"], a["rows"][:, :512], a["o"], _t(16), scale=0.1,
                                                  Sk_max=5, row_index=a["ri"], key_pos=a["kp"], q_pos=a["qp"],
                                                  dk=576, dv=512), name)


def test_noalloc_rejects_sizes_past_the_static_scratch():
    """attn_decode_fwd_noalloc refuses sizes whose split-KV partials exceed the static
    scratch (before any HIP call) and accepts the same checks as attn_decode_fwd."""
    lib = binding.load_library()
    i32 = ctypes.c_int

    def call(B, Hq, Sq, Sk_max):
        return lib.attn_decode_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, 0, 0, 0, B, Hq, 8, Sq, Sk_max, 128, 128,
                                           ctypes.c_float(0.1), 0, ctypes.c_float(0.0), None, FAKE, 64, 512,
                                           FAKE, None, None, None, 0, ctypes.c_int64(0), None, None, None)
    # 256 sequences x 64 heads x 8 draft tokens of up to 32K keys need 68 MB of partials
    assert binding.attn_decode_workspace_bytes(256, 64, 8, 8, 32768, 128, 128) > (64 << 20)
    assert call(256, 64, 8, 32768) == binding.ATTN_ERR_UNSUPPORTED
    assert b"static scratch" in lib.attn_last_error()
    # the ordinary argument checks come first
    assert call(0, 64, 1, 32768) == binding.ATTN_ERR_INVALID_ARG
