"""ctypes binding of libattn.so (argument marshalling only).

Every step of the attention path runs in the library's HIP kernels; this
module checks that tensors are on the GPU with the expected dtype and layout,
reads their sizes, and passes raw device pointers and the current HIP stream.
There is no fallback: if the library is missing or a tensor is not on the
device, the call raises.
"""

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_LOCK = threading.Lock()

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_HIP = 3
ATTN_BF16 = 0
ATTN_F32 = 1
ATTN_F16 = 2
ATTN_Q8_0 = 0
ATTN_Q4_0 = 1
_QFMT = {"q8_0": (ATTN_Q8_0, 34), "q4_0": (ATTN_Q4_0, 18)}


class AttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s (status %d)" % (message, status))
        self.status = status


def library_path():
    return os.environ.get("ATTN_LIBRARY", os.path.join(_HERE, "libattn.so"))


def load_library():
    """Load libattn.so once. torch is imported first so that the library binds to the
    HIP runtime that torch already has in the process."""
    global _LIB
    with _LOCK:
        if _LIB is not None:
            return _LIB
        import torch  # noqa: F401  (HIP runtime first)
        path = library_path()
        if not os.path.exists(path):
            raise AttnError(-1, "libattn.so not found at %s: build it with __graft_entry__.build()" % path)
        lib = ctypes.CDLL(path)
        c_int, c_float, c_void_p, c_size_t = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
        lib.attn_abi_version.restype = c_int
        lib.attn_abi_version.argtypes = []
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_status_string.argtypes = [c_int]
        lib.attn_last_error.restype = ctypes.c_char_p
        lib.attn_last_error.argtypes = []
        lib.attn_prefill_fwd.restype = c_int
        lib.attn_prefill_fwd.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_void_p,
                                         c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                         c_float, c_int, c_float, c_void_p, c_void_p]
        lib.attn_prefill_fwd_ex.restype = c_int
        lib.attn_prefill_fwd_ex.argtypes = [c_void_p, c_int, c_void_p, c_void_p, c_int, c_void_p, c_int, c_void_p,
                                            c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                            c_float, c_int, c_float, c_void_p,
                                            c_void_p, c_int, c_int, ctypes.c_int64, c_float, c_void_p]
        lib.attn_dequant_fp16.restype = c_int
        lib.attn_dequant_fp16.argtypes = [c_void_p, c_int, c_void_p, ctypes.c_int64, c_void_p]
        lib.attn_decode_workspace_bytes.restype = c_size_t
        lib.attn_decode_workspace_bytes.argtypes = [c_int] * 7
        lib.attn_decode_fwd.restype = c_int
        lib.attn_decode_fwd.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                                        c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                        c_float, c_int, c_float, c_void_p,
                                        c_void_p, c_int, c_int, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_int, ctypes.c_int64,
                                        c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        lib.attn_decode_fwd_noalloc.restype = c_int
        lib.attn_decode_fwd_noalloc.argtypes = lib.attn_decode_fwd.argtypes[:-3] + [c_void_p]
        lib.attn_mla_tail_workspace_bytes.restype = c_size_t
        lib.attn_mla_tail_workspace_bytes.argtypes = [c_int] * 5
        lib.attn_mla_tail.restype = c_int
        lib.attn_mla_tail.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                      c_int, c_int, c_int, c_int, c_int, c_void_p, c_size_t, c_void_p]
        _LIB = lib
        return lib


def attn_abi_version():
    return load_library().attn_abi_version()


def attn_status_string(status):
    return load_library().attn_status_string(int(status)).decode()


def _check(status):
    if status != ATTN_OK:
        lib = load_library()
        msg = lib.attn_last_error().decode() or lib.attn_status_string(status).decode()
        raise AttnError(status, msg)


def _ptr(t, name, dtype=None, allow_none=False):
    import torch
    if t is None:
        if allow_none:
            return None
        raise AttnError(ATTN_ERR_INVALID_ARG, "%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise AttnError(ATTN_ERR_INVALID_ARG, "%s must be a torch tensor" % name)
    if t.device.type != "cuda":
        raise AttnError(ATTN_ERR_INVALID_ARG, "%s must be on the GPU (got %s)" % (name, t.device))
    if dtype is not None and t.dtype != dtype:
        raise AttnError(ATTN_ERR_INVALID_ARG, "%s must be %s (got %s)" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise AttnError(ATTN_ERR_INVALID_ARG, "%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _dims(t, name, n):
    """t must be an n-dimensional tensor; returns its shape."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise AttnError(ATTN_ERR_INVALID_ARG, "%s must be a torch tensor" % name)
    if t.dim() != n:
        raise AttnError(ATTN_ERR_INVALID_ARG, "%s must have %d dimensions (got shape %s)" % (name, n, tuple(t.shape)))
    return tuple(int(x) for x in t.shape)


def _expect(t, name, shape):
    """t (if given) must have exactly this shape: the kernels read and write the sizes the
    other tensors define, so a mismatch would run past the end of a buffer."""
    if t is None:
        return
    got = tuple(int(x) for x in t.shape)
    if got != tuple(shape):
        raise AttnError(ATTN_ERR_INVALID_ARG, "%s must have shape %s (got %s)" % (name, tuple(shape), got))


def _row_ptr(t, name):
    """Row array of a gathered cache: rows may be strided, each row contiguous."""
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise AttnError(ATTN_ERR_INVALID_ARG, "%s must be a GPU tensor" % name)
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise AttnError(ATTN_ERR_INVALID_ARG, "%s must be bfloat16 or float16" % name)
    if t.dim() != 2 or t.stride(1) != 1:
        raise AttnError(ATTN_ERR_INVALID_ARG, "%s must be [rows, width] with contiguous rows" % name)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _odtype(o):
    import torch
    if o.dtype == torch.bfloat16:
        return ATTN_BF16
    if o.dtype == torch.float32:
        return ATTN_F32
    raise AttnError(ATTN_ERR_INVALID_ARG, "o must be bfloat16 or float32")


def _qdtype(q):
    import torch
    codes = {torch.bfloat16: ATTN_BF16, torch.float32: ATTN_F32, torch.float16: ATTN_F16}
    if q.dtype not in codes:
        raise AttnError(ATTN_ERR_INVALID_ARG, "q must be bfloat16, float16 or float32")
    return codes[q.dtype]


def _kvdtype(*ts):
    import torch
    codes = {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}
    if any(t.dtype != ts[0].dtype for t in ts) or ts[0].dtype not in codes:
        raise AttnError(ATTN_ERR_INVALID_ARG, "K and V must both be bfloat16 or both float16")
    return codes[ts[0].dtype]


def _prefill_sizes(q, k, v, o, lse, sinks):
    B, Sq, Hq, dk = _dims(q, "q", 4)
    Bk, Sk, Hkv, dkk = _dims(k, "k", 4)
    dv = _dims(v, "v", 4)[3]
    _expect(k, "k", (B, Sk, Hkv, dk))
    _expect(v, "v", (B, Sk, Hkv, dv))
    _expect(o, "o", (B, Sq, Hq, dv))
    _expect(lse, "lse", (B, Hq, Sq))
    _expect(sinks, "sinks", (Hq,))
    return B, Sq, Hq, dk, Sk, Hkv, dv


def attn_prefill_fwd(q, k, v, o, lse=None, *, scale, causal=False, softcap=0.0, sinks=None, stream=None):
    """q [B,Sq,Hq,dk], k [B,Sk,Hkv,dk], v [B,Sk,Hkv,dv] bf16; o [B,Sq,Hq,dv] bf16|fp32;
    lse optional fp32 [B,Hq,Sq]; sinks optional fp32 [Hq]. Enqueued on `stream`
    (default: torch's current stream)."""
    import torch
    lib = load_library()
    B, Sq, Hq, dk, Sk, Hkv, dv = _prefill_sizes(q, k, v, o, lse, sinks)
    st = lib.attn_prefill_fwd(_ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
                              _ptr(v, "v", torch.bfloat16), _ptr(o, "o"), _odtype(o),
                              _ptr(lse, "lse", torch.float32, True),
                              B, Hq, Hkv, Sq, Sk, dk, dv, float(scale), int(bool(causal)), float(softcap),
                              _ptr(sinks, "sinks", torch.float32, True), _stream(stream))
    _check(st)


def attn_prefill_fwd_ex(q, k, v, o, lse=None, *, scale, causal=False, softcap=0.0, sinks=None, mask=None,
                        max_bias=0.0, stream=None):
    """attn_prefill_fwd with q in bf16 / fp16 / fp32 and k, v in bf16 / fp16 (taken from the
    tensors' dtypes), and an optional additive fp16 mask [MB, MH, Sq, W] (contiguous, W >= Sk
    and a multiple of 4; entry [b % MB, h % MH] applies to batch b, head h) times the head's
    ALiBi slope for max_bias."""
    import torch
    lib = load_library()
    B, Sq, Hq, dk, Sk, Hkv, dv = _prefill_sizes(q, k, v, o, lse, sinks)
    mb = mh = 1
    ms = 0
    if mask is not None:
        if mask.dim() != 4 or mask.shape[2] != Sq:
            raise AttnError(ATTN_ERR_INVALID_ARG, "mask must be [MB, MH, Sq, W] (got %s)" % (tuple(mask.shape),))
        mb, mh, ms = int(mask.shape[0]), int(mask.shape[1]), int(mask.shape[3])
    kvt = _kvdtype(k, v)
    st = lib.attn_prefill_fwd_ex(_ptr(q, "q"), _qdtype(q), _ptr(k, "k"), _ptr(v, "v"), kvt,
                                 _ptr(o, "o"), _odtype(o), _ptr(lse, "lse", torch.float32, True),
                                 B, Hq, Hkv, Sq, Sk, dk, dv, float(scale), int(bool(causal)), float(softcap),
                                 _ptr(sinks, "sinks", torch.float32, True),
                                 _ptr(mask, "mask", torch.float16, True), mb, mh, ms, float(max_bias),
                                 _stream(stream))
    _check(st)


def attn_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk_max, dk, dv):
    return int(load_library().attn_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk_max, dk, dv))


def attn_decode_fwd(q, k_cache, v_cache, o, workspace, *, scale, Sk_max, causal=False, softcap=0.0,
                    sinks=None, block_table=None, seq_lens=None, row_index=None, key_pos=None,
                    q_pos=None, kv_row_stride=0, Hkv=None, dk=None, dv=None, k_cur=None, v_cur=None,
                    stream=None):
    """Paged mode: k_cache [n_blocks,Hkv,bs,dk], v_cache [n_blocks,Hkv,bs,dv], block_table
    [B,max_blocks] int32, seq_lens [B] int32. Gathered mode: k_cache / v_cache are 2-D row
    views [rows, width] sharing one row stride (e.g. kv[:, :dk] and kv[:, 64:]), with
    row_index [B,n_sel] int32, key_pos [B,n_sel] fp32, q_pos [B] int32, and optionally the
    tokens' own rows k_cur / v_cur as 2-D row views [B, width] with the same row stride;
    dk defaults to q's width and dv to o's. q [B,Sq,Hq,dk] bf16, o [B,Sq,Hq,dv].
    workspace: a GPU tensor of at least attn_decode_workspace_bytes(...) bytes."""
    lib = load_library()
    args = _decode_args(q, k_cache, v_cache, o, scale, Sk_max, causal, softcap, sinks, block_table, seq_lens,
                        row_index, key_pos, q_pos, kv_row_stride, Hkv, dk, dv, k_cur, v_cur)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.attn_decode_fwd(*args, _ptr(workspace, "workspace"), ws_bytes, _stream(stream)))


def attn_decode_fwd_noalloc(q, k_cache, v_cache, o, *, scale, Sk_max, causal=False, softcap=0.0,
                            sinks=None, block_table=None, seq_lens=None, row_index=None, key_pos=None,
                            q_pos=None, kv_row_stride=0, Hkv=None, dk=None, dv=None, k_cur=None, v_cur=None,
                            stream=None):
    """attn_decode_fwd without a workspace: the split-KV partials go to the library's static
    per-GPU scratch (at most ATTN_NOALLOC_SCRATCH_BYTES; larger sizes raise ATTN_ERR_UNSUPPORTED).
    Calls that overlap on one GPU race; calls ordered on one stream are safe."""
    lib = load_library()
    args = _decode_args(q, k_cache, v_cache, o, scale, Sk_max, causal, softcap, sinks, block_table, seq_lens,
                        row_index, key_pos, q_pos, kv_row_stride, Hkv, dk, dv, k_cur, v_cur)
    _check(lib.attn_decode_fwd_noalloc(*args, _stream(stream)))


def _decode_args(q, k_cache, v_cache, o, scale, Sk_max, causal, softcap, sinks, block_table, seq_lens,
                 row_index, key_pos, q_pos, kv_row_stride, Hkv, dk, dv, k_cur, v_cur):
    """Checked C arguments of a decode call, up to (not including) the workspace."""
    import torch
    B, Sq, Hq, qdk = _dims(q, "q", 4)
    paged = block_table is not None
    if paged:
        n_blocks, Hkv_, bs, dk_ = _dims(k_cache, "k_cache", 4)
        dv_ = _dims(v_cache, "v_cache", 4)[3]
        _expect(v_cache, "v_cache", (n_blocks, Hkv_, bs, dv_))
        Hkv, dk, dv = Hkv_, dk_, dv_
        if qdk != dk:
            raise AttnError(ATTN_ERR_INVALID_ARG, "q's head dim (%d) must equal the key cache's (%d)" % (qdk, dk))
        max_blocks = _dims(block_table, "block_table", 2)[1]
        _expect(block_table, "block_table", (B, max_blocks))
        if seq_lens is None:
            raise AttnError(ATTN_ERR_INVALID_ARG, "paged mode needs seq_lens")
        _expect(seq_lens, "seq_lens", (B,))
        if row_index is not None or k_cur is not None or v_cur is not None:
            raise AttnError(ATTN_ERR_INVALID_ARG, "row_index / k_cur / v_cur belong to gathered mode")
        n_sel = 0
    else:
        bs, max_blocks = 0, 0
        if row_index is None:
            raise AttnError(ATTN_ERR_INVALID_ARG, "give block_table (paged mode) or row_index (gathered mode)")
        n_sel = _dims(row_index, "row_index", 2)[1]
        _expect(row_index, "row_index", (B, n_sel))
        _expect(key_pos, "key_pos", (B, n_sel))
        _expect(q_pos, "q_pos", (B,))
        Hkv = 1 if Hkv is None else Hkv
        dk = qdk if dk is None else dk
        dv = o.shape[3] if dv is None else dv
        if qdk != dk:
            raise AttnError(ATTN_ERR_INVALID_ARG, "q's head dim (%d) must equal dk (%d)" % (qdk, dk))
        if _dims(k_cache, "k_cache", 2)[1] < dk or _dims(v_cache, "v_cache", 2)[1] < dv:
            raise AttnError(ATTN_ERR_INVALID_ARG, "k_cache rows must hold dk and v_cache rows dv elements")
    _expect(o, "o", (B, Sq, Hq, dv))
    _expect(sinks, "sinks", (Hq,))
    if paged:
        kp, vp = _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache")
    else:
        kp, vp = _row_ptr(k_cache, "k_cache"), _row_ptr(v_cache, "v_cache")
        if not kv_row_stride:
            kv_row_stride = k_cache.stride(0)
        if v_cache.stride(0) != kv_row_stride:
            raise AttnError(ATTN_ERR_INVALID_ARG, "k_cache and v_cache rows must share one stride")
        if (k_cur is None) != (v_cur is None):
            raise AttnError(ATTN_ERR_INVALID_ARG, "k_cur and v_cur go together")
        if k_cur is not None:
            kcp, vcp = _row_ptr(k_cur, "k_cur"), _row_ptr(v_cur, "v_cur")
            if k_cur.stride(0) != kv_row_stride or v_cur.stride(0) != kv_row_stride:
                raise AttnError(ATTN_ERR_INVALID_ARG, "k_cur / v_cur rows must have the cache's row stride")
            if k_cur.shape[1] < dk or v_cur.shape[1] < dv:
                raise AttnError(ATTN_ERR_INVALID_ARG, "k_cur rows must hold dk and v_cur rows dv elements")
            if k_cur.shape[0] < B or v_cur.shape[0] < B:
                raise AttnError(ATTN_ERR_INVALID_ARG, "k_cur / v_cur need one row per token")
    if paged or k_cur is None:
        kcp, vcp = None, None
    return (_ptr(q, "q"), kp, vp, _ptr(o, "o"), _odtype(o), _qdtype(q), _kvdtype(k_cache, v_cache),
            B, Hq, Hkv, Sq, int(Sk_max), dk, dv, float(scale), int(bool(causal)),
            float(softcap), _ptr(sinks, "sinks", torch.float32, True),
            _ptr(block_table, "block_table", torch.int32, True), bs, max_blocks,
            _ptr(seq_lens, "seq_lens", torch.int32, True),
            _ptr(row_index, "row_index", torch.int32, True),
            _ptr(key_pos, "key_pos", torch.float32, True),
            _ptr(q_pos, "q_pos", torch.int32, True), n_sel, int(kv_row_stride),
            kcp, vcp)


def attn_dequant_fp16(src, fmt, dst, stream=None):
    """src: uint8 GPU tensor of packed blocks ("q8_0": 34 bytes, "q4_0": 18 bytes per 32
    values); dst: float16 GPU tensor with 32 elements per block. Enqueued on `stream`."""
    import torch
    lib = load_library()
    code, size = _QFMT[fmt]
    if src.dtype != torch.uint8 or src.numel() % size:
        raise AttnError(ATTN_ERR_INVALID_ARG, "src must be uint8 holding whole %s blocks" % fmt)
    n = src.numel() // size
    if dst.dtype != torch.float16 or dst.numel() != 32 * n:
        raise AttnError(ATTN_ERR_INVALID_ARG, "dst must be float16 with 32 elements per block")
    _check(lib.attn_dequant_fp16(_ptr(src, "src"), code, _ptr(dst, "dst"), n, _stream(stream)))


def attn_mla_tail_workspace_bytes(T, H, R, DV, N):
    return int(load_library().attn_mla_tail_workspace_bytes(T, H, R, DV, N))


def attn_mla_tail(o_lat, w_absorb, w_o, y, workspace, stream=None):
    """MLA decode tail. o_lat bf16 [T, H, R] (or [T, 1, H, R]), w_absorb bf16 [H, DV, R],
    w_o bf16 [H*DV, N], y [T, N] bf16 or float32, workspace a uint8 GPU tensor of at least
    attn_mla_tail_workspace_bytes(T, H, R, DV, N) bytes. Enqueued on `stream`."""
    import torch
    lib = load_library()
    if w_absorb.dim() != 3 or w_o.dim() != 2 or y.dim() != 2:
        raise AttnError(ATTN_ERR_INVALID_ARG, "w_absorb must be [H, DV, R], w_o [H*DV, N] and y [T, N]")
    H, DV, R = w_absorb.shape
    N = w_o.shape[1]
    T = y.shape[0]
    if o_lat.numel() != T * H * R or w_o.shape[0] != H * DV or y.shape[1] != N:
        raise AttnError(ATTN_ERR_INVALID_ARG, "shape mismatch: o_lat %s, w_absorb %s, w_o %s, y %s" %
                        (tuple(o_lat.shape), tuple(w_absorb.shape), tuple(w_o.shape), tuple(y.shape)))
    ycode = _odtype(y)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.attn_mla_tail(_ptr(o_lat, "o_lat", torch.bfloat16), _ptr(w_absorb, "w_absorb", torch.bfloat16),
                             _ptr(w_o, "w_o", torch.bfloat16), _ptr(y, "y"), ycode, T, H, R, DV, N,
                             _ptr(workspace, "workspace"), ws_bytes, _stream(stream)))
