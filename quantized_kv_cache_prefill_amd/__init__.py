"""Python binding of libkvq4.so -- int4 group-wise KV cache and decode attention on MI355X.

Argument marshalling only: every step of the path runs in the HIP kernels of
``csrc/``.  PyTorch supplies device memory and the current stream.  The
functions mirror the C entry points declared in ``include/kvq4.h`` (same
names, same semantics); see that header for the operation each one performs
and the passage of the FlexGen pages it follows.

If ``libkvq4.so`` has not been built, importing works but every call raises
``RuntimeError`` -- there is no CPU fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

__all__ = [
    "KvqError", "QuantKVCache", "kvq_cache_bytes", "kvq_workspace_bytes", "kv_quantize_prefill",
    "kv_append_quant", "decode_attention_q4", "decode_attention_q4_tuned", "kv_append_attend_q4",
    "decode_attention_q4_topk", "decode_attention_q4_noalloc", "kvq_w4_quantize", "kvq_gemm_w4_workspace_bytes", "gemm_w4a16",
    "kv_quantize_prefill_host", "kv_append_quant_host", "decode_attention_q4_host", "kvq_host_simd",
    "kvq_host_use_simd", "kvq_stream_read", "kvq_codec_params",
    "library_path", "load_library", "GROUP",
]

GROUP = 64
META_F32 = 0
META_F16 = 1
_META = {"f32": (META_F32, torch.float32), "f16": (META_F16, torch.float16)}
KVQ_TOPK_MAX_CTX = 8192
KVQ_TOPK_FUSED_MAX_CTX = 2048
KVQ_MAX_SPLITS = 256
KVQ_GEMM_STREAM = -1  # gemm_w4a16 num_splits: the stream form

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvq4.so")

EXPORTED = ("kvq_cache_bytes", "kv_quantize_prefill", "kv_quantize_prefill_attend", "kv_append_quant", "kvq_workspace_bytes",
            "decode_attention_q4", "decode_attention_q4_tuned", "kv_append_attend_q4", "decode_attention_q4_topk",
            "decode_attention_q4_noalloc",
            "kvq_w4_quantize", "kvq_gemm_w4_workspace_bytes", "gemm_w4a16", "kv_quantize_prefill_host",
            "kv_append_quant_host", "decode_attention_q4_host", "kvq_host_simd", "kvq_host_use_simd", "kvq_strerror",
            "kvq_stream_read", "kvq_codec_params")


class KvqDims(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int32), ("a", ctypes.c_int32), ("h", ctypes.c_int32), ("s", ctypes.c_int32),
                ("n", ctypes.c_int32), ("group", ctypes.c_int32), ("meta_dtype", ctypes.c_int32)]


class KvqCache(ctypes.Structure):
    _fields_ = [("dims", KvqDims), ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_min", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v_min", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p)]


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({_strerror(status)})")


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libkvq4.so (raises RuntimeError when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m quantized_kv_cache_prefill_amd.build`"
                           " (there is no CPU fallback)")
    L = ctypes.CDLL(_LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    PD, PC = ctypes.POINTER(KvqDims), ctypes.POINTER(KvqCache)
    L.kvq_cache_bytes.argtypes = [PD, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
    L.kvq_cache_bytes.restype = ctypes.c_int
    L.kv_quantize_prefill.argtypes = [PC, P, P, I32, P]
    L.kv_quantize_prefill.restype = ctypes.c_int
    L.kv_quantize_prefill_attend.argtypes = [PC, P, P, P, I32, P, P]
    L.kv_quantize_prefill_attend.restype = ctypes.c_int
    L.kv_append_quant.argtypes = [PC, P, P, I32, P]
    L.kv_append_quant.restype = ctypes.c_int
    L.kvq_workspace_bytes.argtypes = [PD, I32, I32, I32]
    L.kvq_workspace_bytes.restype = SZ
    L.decode_attention_q4.argtypes = [PC, P, I32, P, I32, P, SZ, P]
    L.decode_attention_q4.restype = ctypes.c_int
    L.decode_attention_q4_tuned.argtypes = [PC, P, I32, P, I32, I32, I32, P, SZ, P]
    L.decode_attention_q4_tuned.restype = ctypes.c_int
    L.kv_append_attend_q4.argtypes = [PC, P, P, P, I32, P, I32, P, SZ, P]
    L.kv_append_attend_q4.restype = ctypes.c_int
    L.decode_attention_q4_noalloc.argtypes = [PC, P, I32, P, I32, P]
    L.decode_attention_q4_noalloc.restype = ctypes.c_int
    L.decode_attention_q4_topk.argtypes = [PC, P, I32, I32, P, P, P, SZ, P]
    L.decode_attention_q4_topk.restype = ctypes.c_int
    L.kvq_w4_quantize.argtypes = [P, I32, I32, P, P, P, P]
    L.kvq_w4_quantize.restype = ctypes.c_int
    L.kvq_gemm_w4_workspace_bytes.argtypes = [I32, I32, I32, I32]
    L.kvq_gemm_w4_workspace_bytes.restype = SZ
    L.gemm_w4a16.argtypes = [P, I32, I32, I32, P, P, P, P, I32, P, SZ, P]
    L.gemm_w4a16.restype = ctypes.c_int
    L.kv_quantize_prefill_host.argtypes = [PC, P, P, I32, I32]
    L.kv_quantize_prefill_host.restype = ctypes.c_int
    L.kv_append_quant_host.argtypes = [PC, P, P, I32, I32]
    L.kv_append_quant_host.restype = ctypes.c_int
    L.decode_attention_q4_host.argtypes = [PC, P, I32, P, I32]
    L.decode_attention_q4_host.restype = ctypes.c_int
    L.kvq_host_simd.argtypes = []
    L.kvq_host_simd.restype = ctypes.c_int
    L.kvq_host_use_simd.argtypes = [ctypes.c_int]
    L.kvq_host_use_simd.restype = None
    L.kvq_stream_read.argtypes = [P, SZ, P, P]
    L.kvq_stream_read.restype = ctypes.c_int
    L.kvq_codec_params.argtypes = [P, ctypes.c_int64, ctypes.c_int, P, P, P]
    L.kvq_codec_params.restype = ctypes.c_int
    L.kvq_strerror.argtypes = [ctypes.c_int]
    L.kvq_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def _strerror(status: int) -> str:
    try:
        return load_library().kvq_strerror(status).decode()
    except Exception:  # noqa: BLE001 - only used to format an error message
        return "?"


def _check(status: int, what: str):
    if status != 0:
        raise KvqError(status, what)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Allocation context for the buffers a call creates itself (workspace, out, sel_idx):
    on the stream its kernels run on, so that the caching allocator ties each block to that
    stream and never hands it to work on another stream while the kernels may still use it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def make_dims(b: int, a: int, h: int, s: int, n: int, meta: str = "f32") -> KvqDims:
    return KvqDims(b, a, h, s, n, GROUP, _META[meta][0])


class QuantKVCache:
    """One layer's int4 KV cache in device memory (planes owned by torch).

    k_codes, v_codes : uint8   [b, a, S, d/2]   (two codes per byte, even element low nibble)
    k_min, k_scale, v_min, v_scale : float32 (meta="f32") or float16 (meta="f16") [b, a, S, d/64]
    with S = s + n slots, d = h / a.
    """

    def __init__(self, b: int, a: int, h: int, s: int, n: int, device="cuda", fill: int | None = None,
                 meta: str = "f32"):
        if h % a != 0:
            raise ValueError("h must be a multiple of a")
        if meta not in _META:
            raise ValueError("meta must be 'f32' or 'f16'")
        self.meta = meta
        self.b, self.a, self.h, self.s, self.n = b, a, h, s, n
        self.d = h // a
        self.S = s + n
        G = self.d // GROUP
        alloc = torch.empty if fill is None else (lambda *sh, **kw: torch.full(sh, fill, **kw))
        self.k_codes = alloc(b, a, self.S, self.d // 2, dtype=torch.uint8, device=device)
        self.v_codes = alloc(b, a, self.S, self.d // 2, dtype=torch.uint8, device=device)
        planes = [alloc(b, a, self.S, G, dtype=_META[meta][1], device=device) for _ in range(4)]
        self.k_min, self.k_scale, self.v_min, self.v_scale = planes
        self._struct = KvqCache(make_dims(b, a, h, s, n, meta), self.k_codes.data_ptr(), self.v_codes.data_ptr(),
                                self.k_min.data_ptr(), self.k_scale.data_ptr(), self.v_min.data_ptr(),
                                self.v_scale.data_ptr())

    @property
    def dims(self) -> KvqDims:
        return self._struct.dims

    def struct_ref(self):
        return ctypes.byref(self._struct)

    def planes(self):
        return (self.k_codes, self.k_min, self.k_scale, self.v_codes, self.v_min, self.v_scale)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.planes())


def _act(t: torch.Tensor, shape, name: str):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or not t.is_cuda:
        raise TypeError(f"{name} must be a float16 CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def kvq_cache_bytes(b: int, a: int, h: int, s: int, n: int, meta: str = "f32") -> tuple[int, int]:
    """(bytes of one code plane, bytes of one metadata plane)."""
    cb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().kvq_cache_bytes(ctypes.byref(make_dims(b, a, h, s, n, meta)), ctypes.byref(cb),
                                          ctypes.byref(mb)), "kvq_cache_bytes")
    return cb.value, mb.value


def kvq_workspace_bytes(cache: QuantKVCache, ctx_len: int, num_splits: int = 0, k_top: int = 0) -> int:
    return load_library().kvq_workspace_bytes(ctypes.byref(cache.dims), ctx_len, num_splits, k_top)


def kv_quantize_prefill(cache: QuantKVCache, k: torch.Tensor, v: torch.Tensor, stream=None):
    """Quantise the prompt's K and V (fp16 [b, s_len, a, d]) into slots 0..s_len-1."""
    s_len = k.shape[1] if k.dim() == 4 else -1
    _act(k, (cache.b, s_len, cache.a, cache.d), "k")
    _act(v, (cache.b, s_len, cache.a, cache.d), "v")
    _check(load_library().kv_quantize_prefill(cache.struct_ref(), _ptr(k), _ptr(v), s_len, _stream(stream)),
           "kv_quantize_prefill")


def kv_quantize_prefill_attend(cache: QuantKVCache, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One launch: the planes of kv_quantize_prefill for slots 0..s_len-1 and the causal
    prefill attention softmax(q k^T / sqrt(d)) v over the fp16 prompt; q, k, v, out fp16
    [b, s_len, a, d]."""
    s_len = k.shape[1] if k.dim() == 4 else -1
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _act(t, (cache.b, s_len, cache.a, cache.d), name)
    out = _out_like(q, out, stream)
    _act(out, q.shape, "out")
    _check(load_library().kv_quantize_prefill_attend(cache.struct_ref(), _ptr(q), _ptr(k), _ptr(v), s_len, _ptr(out),
                                                     _stream(stream)), "kv_quantize_prefill_attend")
    return out


def kv_append_quant(cache: QuantKVCache, k_new: torch.Tensor, v_new: torch.Tensor, pos: int, stream=None):
    """Quantise one new token's K and V (fp16 [b, 1, a, d]) into slot `pos`."""
    _act(k_new, (cache.b, 1, cache.a, cache.d), "k_new")
    _act(v_new, (cache.b, 1, cache.a, cache.d), "v_new")
    _check(load_library().kv_append_quant(cache.struct_ref(), _ptr(k_new), _ptr(v_new), pos, _stream(stream)),
           "kv_append_quant")


def _workspace(cache, ctx_len, num_splits, ws, stream):
    need = kvq_workspace_bytes(cache, ctx_len, num_splits)
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        with _on(stream):
            ws = torch.empty(need // 4, dtype=torch.float32, device=cache.k_codes.device)
    return ws, need


def _out_like(q: torch.Tensor, out, stream):
    if out is None:
        with _on(stream):
            out = torch.empty_like(q)
    return out


def decode_attention_q4(cache: QuantKVCache, q: torch.Tensor, ctx_len: int, out: torch.Tensor | None = None,
                        num_splits: int = 0, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """softmax(q K^T / sqrt(d)) V over slots 0..ctx_len-1; q, out fp16 [b, 1, a, d]."""
    _act(q, (cache.b, 1, cache.a, cache.d), "q")
    out = _out_like(q, out, stream)
    _act(out, q.shape, "out")
    ws, need = _workspace(cache, ctx_len, num_splits, ws, stream)
    _check(load_library().decode_attention_q4(cache.struct_ref(), _ptr(q), ctx_len, _ptr(out), num_splits,
                                              _ptr(ws), need, _stream(stream)), "decode_attention_q4")
    return out


def decode_attention_q4_tuned(cache: QuantKVCache, q: torch.Tensor, ctx_len: int, unroll: int,
                              waves_per_pair: int, out: torch.Tensor | None = None, num_splits: int = 0,
                              ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """decode_attention_q4 with an explicit kernel launch shape (unroll 1/2/4, waves per pair 1/2/4)."""
    _act(q, (cache.b, 1, cache.a, cache.d), "q")
    out = _out_like(q, out, stream)
    _act(out, q.shape, "out")
    ws, need = _workspace(cache, ctx_len, num_splits, ws, stream)
    _check(load_library().decode_attention_q4_tuned(cache.struct_ref(), _ptr(q), ctx_len, _ptr(out), num_splits,
                                                    unroll, waves_per_pair, _ptr(ws), need, _stream(stream)),
           "decode_attention_q4_tuned")
    return out


KVQ_NOALLOC_SCRATCH_BYTES = 32 << 20


def decode_attention_q4_noalloc(cache: QuantKVCache, q: torch.Tensor, ctx_len: int, out: torch.Tensor,
                                num_splits: int = 0, stream=None) -> torch.Tensor:
    """decode_attention_q4 with its split partials in the library's static device workspace:
    nothing is allocated, here or in the library; the caller passes `out`.  Raises KvqError
    (KVQ_ENOSPACE) when the launch needs more than KVQ_NOALLOC_SCRATCH_BYTES of partials.
    Calls that may overlap on one GPU race on that workspace."""
    _act(q, (cache.b, 1, cache.a, cache.d), "q")
    _act(out, q.shape, "out")
    _check(load_library().decode_attention_q4_noalloc(cache.struct_ref(), _ptr(q), ctx_len, _ptr(out), num_splits,
                                                      _stream(stream)), "decode_attention_q4_noalloc")
    return out


def kv_append_attend_q4(cache: QuantKVCache, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, pos: int,
                        out: torch.Tensor | None = None, num_splits: int = 0, ws: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """One decode step in one launch: append (k_new, v_new) at slot `pos`, then attend over
    slots 0..pos with q.  All fp16 [b, 1, a, d]."""
    for t, name in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
        _act(t, (cache.b, 1, cache.a, cache.d), name)
    out = _out_like(q, out, stream)
    _act(out, q.shape, "out")
    ws, need = _workspace(cache, pos + 1, num_splits, ws, stream)
    _check(load_library().kv_append_attend_q4(cache.struct_ref(), _ptr(q), _ptr(k_new), _ptr(v_new), pos, _ptr(out),
                                              num_splits, _ptr(ws), need, _stream(stream)), "kv_append_attend_q4")
    return out


def decode_attention_q4_topk(cache: QuantKVCache, q: torch.Tensor, ctx_len: int, k_top: int,
                             out: torch.Tensor | None = None, sel_idx: torch.Tensor | bool | None = True,
                             ws: torch.Tensor | None = None, stream=None):
    """Top-k sparse decode attention.  Returns (out fp16 [b,1,a,d], sel_idx int32 [b,a,k_top] or None)."""
    _act(q, (cache.b, 1, cache.a, cache.d), "q")
    out = _out_like(q, out, stream)
    _act(out, q.shape, "out")
    if sel_idx is True:
        with _on(stream):
            sel_idx = torch.empty((cache.b, cache.a, k_top), dtype=torch.int32, device=q.device)
    elif sel_idx is False:
        sel_idx = None
    if sel_idx is not None and (sel_idx.dtype != torch.int32 or not sel_idx.is_contiguous()
                                or sel_idx.numel() != cache.b * cache.a * k_top):
        raise ValueError("sel_idx must be a contiguous int32 tensor of b*a*k_top elements")
    # ws: the scores; optional up to KVQ_TOPK_FUSED_MAX_CTX tokens (a ws that is given receives them)
    need = kvq_workspace_bytes(cache, ctx_len, 0, k_top)
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        with _on(stream):
            ws = torch.empty(need // 4, dtype=torch.float32, device=q.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().decode_attention_q4_topk(cache.struct_ref(), _ptr(q), ctx_len, k_top, _ptr(out),
                                                   _ptr(sel_idx), _ptr(ws), ws_bytes, _stream(stream)),
           "decode_attention_q4_topk")
    return out, sel_idx


# ------------------------------------------------------------ int4 weights
def _t16(t: torch.Tensor, shape, name: str):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float16 CUDA tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def kvq_w4_quantize(w: torch.Tensor, stream=None):
    """W fp16 [N, K] -> device planes in the tiled layout gemm_w4a16 streams:
    codes uint8 [N/64, K/128, 64, 64], mins and scales fp16 [N/64, K/128, 64, 2]
    (tile (nt, kt): rows 64nt.., k 128kt..; row r, k-byte j; row r, group h)."""
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    N, K = w.shape
    _t16(w, (N, K), "w")
    if N % 64 or K % 128:
        raise ValueError("N must be a multiple of 64 and K of 128")
    with _on(stream):
        codes = torch.empty((N // 64, K // 128, 64, 64), dtype=torch.uint8, device=w.device)
        mins = torch.empty((N // 64, K // 128, 64, 2), dtype=torch.float16, device=w.device)
        scales = torch.empty_like(mins)
    _check(load_library().kvq_w4_quantize(_ptr(w), N, K, _ptr(codes), _ptr(mins), _ptr(scales), _stream(stream)),
           "kvq_w4_quantize")
    return codes, mins, scales


def kvq_gemm_w4_workspace_bytes(M: int, N: int, K: int, num_splits: int = 0) -> int:
    return load_library().kvq_gemm_w4_workspace_bytes(M, N, K, num_splits)


def gemm_w4a16(x: torch.Tensor, codes: torch.Tensor, mins: torch.Tensor, scales: torch.Tensor,
               y: torch.Tensor | None = None, num_splits: int = 0, ws: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """y = x W^T with int4 weights in the tiled layout of kvq_w4_quantize: x fp16 [M, K] -> y fp16 [M, N]."""
    if x.dim() != 2 or codes.dim() != 4:
        raise ValueError("x must be [M, K] and codes [N/64, K/128, 64, 64]")
    M, K = x.shape
    N = codes.shape[0] * 64
    _t16(x, (M, K), "x")
    if (codes.dtype != torch.uint8 or not codes.is_contiguous()
            or tuple(codes.shape) != (N // 64, K // 128, 64, 64)):
        raise ValueError("codes must be a contiguous uint8 tensor [N/64, K/128, 64, 64]")
    _t16(mins, (N // 64, K // 128, 64, 2), "mins")
    _t16(scales, (N // 64, K // 128, 64, 2), "scales")
    if y is None:
        with _on(stream):
            y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _t16(y, (M, N), "y")
    need = kvq_gemm_w4_workspace_bytes(M, N, K, num_splits)
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        with _on(stream):
            ws = torch.empty(need // 4, dtype=torch.float32, device=x.device)
    _check(load_library().gemm_w4a16(_ptr(x), M, N, K, _ptr(codes), _ptr(mins), _ptr(scales), _ptr(y), num_splits,
                                     _ptr(ws), need, _stream(stream)), "gemm_w4a16")
    return y


# --------------------------------------------------------------- measurement
def kvq_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Read every byte of the device tensor `buf` once (the HBM read ceiling); `sink` is a
    uint32/int32 device tensor of at least ceil(nbytes / 65536) elements."""
    nbytes = buf.numel() * buf.element_size()
    if not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous CUDA tensor")
    if sink.element_size() != 4 or not sink.is_cuda or sink.numel() < (nbytes + 65535) // 65536:
        raise ValueError("sink must be a 4-byte CUDA tensor of ceil(nbytes/65536) elements")
    _check(load_library().kvq_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "kvq_stream_read")


def kvq_codec_params(rng: torch.Tensor, meta: str = "f32", scale: torch.Tensor | None = None,
                     inv: torch.Tensor | None = None, stream=None):
    """The codec's stored scale and inverse scale (binary32) for each range in the float32
    CUDA tensor `rng` (all > 0), as every quantiser of this library computes them."""
    if not rng.is_cuda or rng.dtype != torch.float32 or not rng.is_contiguous():
        raise TypeError("rng must be a contiguous float32 CUDA tensor")
    scale = _out_like(rng, scale, stream)
    inv = _out_like(rng, inv, stream)
    for t, name in ((scale, "scale"), (inv, "inv")):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != rng.numel():
            raise TypeError(f"{name} must be a contiguous float32 CUDA tensor of rng's size")
    _check(load_library().kvq_codec_params(_ptr(rng), rng.numel(), _META[meta][0], _ptr(scale), _ptr(inv),
                                           _stream(stream)), "kvq_codec_params")
    return scale, inv


# ------------------------------------------------------------------ host path
def _host(t: torch.Tensor, shape, name: str):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float16 CPU tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _host_cache(cache: QuantKVCache):
    if cache.k_codes.is_cuda:
        raise TypeError("the host calls need a cache in CPU memory (QuantKVCache(..., device='cpu'))")


def kv_quantize_prefill_host(cache: QuantKVCache, k: torch.Tensor, v: torch.Tensor, n_threads: int = 0):
    """kv_quantize_prefill on the CPU: cache and fp16 [b, s_len, a, d] inputs in host memory."""
    _host_cache(cache)
    s_len = k.shape[1] if k.dim() == 4 else -1
    _host(k, (cache.b, s_len, cache.a, cache.d), "k")
    _host(v, (cache.b, s_len, cache.a, cache.d), "v")
    _check(load_library().kv_quantize_prefill_host(cache.struct_ref(), _ptr(k), _ptr(v), s_len, n_threads),
           "kv_quantize_prefill_host")


def kv_append_quant_host(cache: QuantKVCache, k_new: torch.Tensor, v_new: torch.Tensor, pos: int,
                         n_threads: int = 0):
    _host_cache(cache)
    _host(k_new, (cache.b, 1, cache.a, cache.d), "k_new")
    _host(v_new, (cache.b, 1, cache.a, cache.d), "v_new")
    _check(load_library().kv_append_quant_host(cache.struct_ref(), _ptr(k_new), _ptr(v_new), pos, n_threads),
           "kv_append_quant_host")


def decode_attention_q4_host(cache: QuantKVCache, q: torch.Tensor, ctx_len: int, out: torch.Tensor | None = None,
                             n_threads: int = 0) -> torch.Tensor:
    """decode_attention_q4 on the CPU over a host-resident cache; q, out fp16 [b, 1, a, d] in host memory."""
    _host_cache(cache)
    _host(q, (cache.b, 1, cache.a, cache.d), "q")
    if out is None:
        out = torch.empty_like(q)
    _host(out, q.shape, "out")
    _check(load_library().decode_attention_q4_host(cache.struct_ref(), _ptr(q), ctx_len, _ptr(out), n_threads),
           "decode_attention_q4_host")
    return out


def kvq_host_simd() -> bool:
    return bool(load_library().kvq_host_simd())


def kvq_host_use_simd(enable: bool):
    load_library().kvq_host_use_simd(1 if enable else 0)
