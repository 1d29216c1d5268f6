"""CPU oracle for the int4 group-wise KV cache and int4-cache decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never imports, links or calls it, and it imports nothing from the library.

The arithmetic lives in ``kvq_oracle.c`` (plain scalar C, built with gcc
``-O2 -ffp-contract=off``, no fast-math).  This module only builds that file
and marshals numpy arrays into it.  What each function computes and which
page passage it follows is stated in the C source:

* codec -- "FlexGen研究学术报告", section 三.2(C): group-wise asymmetric
  4-bit quantisation, 64 contiguous elements per group, with binary32 or
  binary16 (``*_m16``) min/scale planes; attention uses the
  dequantised values min + code*scale exactly (the report's FP16 form is
  available as ``dequant_rows_f16``);
* dense attention -- the FlexGen blog's decode-phase equation (section
  "解码阶段") with the 1/sqrt(d_k) scale of the efficient-inference survey's
  eq. (2);
* top-k sparse attention -- the same report section's top-10% sparse
  attention;
* prefill attention -- the blog's prefill-phase equation (section
  "预填充阶段"), causal, over the fp16 K and V.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")
GROUP = 64

_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-frounding-math", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile kvq_oracle.c into libkvq_oracle.so with gcc."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(L: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    I = ctypes.c_int
    L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_f16_to_f32.restype = ctypes.c_float
    L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    L.oracle_f32_to_f16.restype = ctypes.c_uint16
    L.oracle_quantize_group.argtypes = [P, P, P, P]
    L.oracle_quantize_rows.argtypes = [I, I, P, P, P, P]
    L.oracle_quantize_group_m16.argtypes = [P, P, P, P]
    L.oracle_w_dequant.argtypes = [I, ctypes.c_uint16, ctypes.c_uint16]
    L.oracle_w_dequant.restype = ctypes.c_uint16
    L.oracle_gemm_w4a16.argtypes = [I, I, I, P, P, P, P, P]
    L.oracle_gemm_w4a16.restype = None
    L.oracle_quantize_rows_m16.argtypes = [I, I, P, P, P, P]
    L.oracle_dequant_rows.argtypes = [I, I, P, P, P, P]
    L.oracle_dequant_rows_f16.argtypes = [I, I, P, P, P, P]
    L.oracle_scores.argtypes = [I, I, P, P, P, P, P]
    L.oracle_attend.argtypes = [I, I, P, P, P, P, P, P, P, P]
    L.oracle_attend_subset.argtypes = [I, I, P, P, P, P, P, P, P, P, P]
    L.oracle_select_topk.argtypes = [I, P, I, P]
    L.oracle_attend_topk.argtypes = [I, I, I, P, P, P, P, P, P, P, P, P]
    L.oracle_prefill_attend.argtypes = [I, I, I, P, P, P, P]
    L.oracle_attend_rows.argtypes = [I, I, P, P, P, P]
    L.oracle_prefill_attend_rows.argtypes = [I, I, I, P, P, P, I, P, P]
    L.oracle_codec_params.argtypes = [I, ctypes.c_int64, P, P, P]
    for f in ("oracle_quantize_group", "oracle_quantize_rows", "oracle_quantize_group_m16", "oracle_quantize_rows_m16",
              "oracle_dequant_rows", "oracle_dequant_rows_f16",
              "oracle_scores",
              "oracle_attend", "oracle_attend_subset", "oracle_select_topk", "oracle_attend_topk",
              "oracle_attend_rows", "oracle_prefill_attend", "oracle_prefill_attend_rows", "oracle_codec_params"):
        getattr(L, f).restype = None
    return L


_lib = None
_override = None


def lib() -> ctypes.CDLL:
    """The loaded oracle library (a test may swap in another build with use_library)."""
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


class use_library:
    """Context manager: route every oracle call through the shared object at ``path``.

    Used only by the tests that plant a mistake in a copy of the oracle source to
    show that the pins catch it.
    """

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _override
        self._prev = _override
        _override = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _override
        _override = self._prev
        return False


def compile_variant(source_text: str, out_path: str) -> str:
    """Compile C source text with the oracle's own flags (for planted-mistake tests)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.check_call(["gcc", *_CFLAGS, "-w", "-o", out_path, src, "-lm"])
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _f16bits(x) -> np.ndarray:
    """fp16 array (or its uint16 bit pattern) -> contiguous uint16 bits."""
    x = np.asarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    assert x.dtype == np.uint16, x.dtype
    return np.ascontiguousarray(x)


# ---------------------------------------------------------------- conversions
def f16_to_f32(bits: int) -> float:
    return lib().oracle_f16_to_f32(int(bits))


def f32_to_f16(x: float) -> int:
    return lib().oracle_f32_to_f16(float(x))


# --------------------------------------------------------------------- codec
def quantize_group(x64):
    """One group of 64 fp16 values -> (codes uint8[32], min float32, scale float32)."""
    x = _f16bits(x64).reshape(-1)
    assert x.size == GROUP
    codes = np.zeros(GROUP // 2, np.uint8)
    mn = np.zeros(1, np.float32)
    sc = np.zeros(1, np.float32)
    lib().oracle_quantize_group(_ptr(x), _ptr(codes), _ptr(mn), _ptr(sc))
    return codes, mn[0], sc[0]


def codec_params(rng, meta: str = "f32"):
    """The codec's stored scale (widened to float32) and inverse for each group range in the
    float32 array `rng` (all > 0), binary32 (meta "f32") or binary16 ("f16") metadata."""
    r = np.ascontiguousarray(rng, dtype=np.float32).reshape(-1)
    scale = np.empty_like(r)
    inv = np.empty_like(r)
    lib().oracle_codec_params(1 if meta == "f16" else 0, r.size, _ptr(r), _ptr(scale), _ptr(inv))
    return scale, inv


def quantize_rows(x):
    """x: fp16 [..., d] (d a multiple of 64).  Every row is quantised on its own.

    Returns codes uint8 [..., d/2], mins float32 [..., d/64], scales float32 [..., d/64].
    """
    x = _f16bits(x)
    d = x.shape[-1]
    assert d % GROUP == 0
    lead = x.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    codes = np.zeros(lead + (d // 2,), np.uint8)
    mins = np.zeros(lead + (d // GROUP,), np.float32)
    scales = np.zeros(lead + (d // GROUP,), np.float32)
    lib().oracle_quantize_rows(n, d, _ptr(x), _ptr(codes), _ptr(mins), _ptr(scales))
    return codes, mins, scales


def quantize_group_m16(x64):
    """One group with binary16 metadata -> (codes uint8[32], min float16, scale float16)."""
    x = _f16bits(x64).reshape(-1)
    assert x.size == GROUP
    codes = np.zeros(GROUP // 2, np.uint8)
    mn = np.zeros(1, np.uint16)
    sc = np.zeros(1, np.uint16)
    lib().oracle_quantize_group_m16(_ptr(x), _ptr(codes), _ptr(mn), _ptr(sc))
    return codes, mn.view(np.float16)[0], sc.view(np.float16)[0]


def quantize_rows_m16(x):
    """Like quantize_rows with binary16 metadata: mins/scales float16 [..., d/64]."""
    x = _f16bits(x)
    d = x.shape[-1]
    assert d % GROUP == 0
    lead = x.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    codes = np.zeros(lead + (d // 2,), np.uint8)
    mins = np.zeros(lead + (d // GROUP,), np.uint16)
    scales = np.zeros(lead + (d // GROUP,), np.uint16)
    lib().oracle_quantize_rows_m16(n, d, _ptr(x), _ptr(codes), _ptr(mins), _ptr(scales))
    return codes, mins.view(np.float16), scales.view(np.float16)


def _dequant_args(codes, mins, scales):
    codes = np.ascontiguousarray(codes, np.uint8)
    mins = np.ascontiguousarray(mins, np.float32)
    scales = np.ascontiguousarray(scales, np.float32)
    d = codes.shape[-1] * 2
    lead = codes.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    return codes, mins, scales, d, lead, n


def dequant_rows(codes, mins, scales) -> np.ndarray:
    """Dequantised values min + code*scale (float64): codes [..., d/2], mins/scales [..., d/64] -> [..., d]."""
    codes, mins, scales, d, lead, n = _dequant_args(codes, mins, scales)
    out = np.zeros(lead + (d,), np.float64)
    lib().oracle_dequant_rows(n, d, _ptr(codes), _ptr(mins), _ptr(scales), _ptr(out))
    return out


def dequant_rows_f16(codes, mins, scales) -> np.ndarray:
    """The report's FP16 form of the dequantised values (float16 [..., d]); reference only."""
    codes, mins, scales, d, lead, n = _dequant_args(codes, mins, scales)
    out = np.zeros(lead + (d,), np.uint16)
    lib().oracle_dequant_rows_f16(n, d, _ptr(codes), _ptr(mins), _ptr(scales), _ptr(out))
    return out.view(np.float16)


# ----------------------------------------------------------------- attention
class HeadCache:
    """Quantised cache of ONE (batch row, head): codes [T][d/2], mins/scales [T][d/64]."""

    def __init__(self, k_codes, k_min, k_scale, v_codes, v_min, v_scale):
        self.kc = np.ascontiguousarray(k_codes, np.uint8)
        self.kmin = np.ascontiguousarray(k_min, np.float32)
        self.ksc = np.ascontiguousarray(k_scale, np.float32)
        self.vc = np.ascontiguousarray(v_codes, np.uint8)
        self.vmin = np.ascontiguousarray(v_min, np.float32)
        self.vsc = np.ascontiguousarray(v_scale, np.float32)
        self.d = self.kc.shape[-1] * 2
        self.T = self.kc.shape[0]

    def kargs(self):
        return _ptr(self.kc), _ptr(self.kmin), _ptr(self.ksc)

    def vargs(self):
        return _ptr(self.vc), _ptr(self.vmin), _ptr(self.vsc)


def scores(q, hc: HeadCache, T: int | None = None) -> np.ndarray:
    T = hc.T if T is None else T
    q = _f16bits(q).reshape(-1)
    s = np.zeros(T, np.float64)
    lib().oracle_scores(hc.d, T, _ptr(q), *hc.kargs(), _ptr(s))
    return s


def attend(q, hc: HeadCache, T: int | None = None) -> np.ndarray:
    """Dense decode attention of one (batch row, head) over tokens 0..T-1 (fp64 result)."""
    T = hc.T if T is None else T
    assert 1 <= T <= hc.T
    q = _f16bits(q).reshape(-1)
    out = np.zeros(hc.d, np.float64)
    lib().oracle_attend(hc.d, T, _ptr(q), *hc.kargs(), *hc.vargs(), _ptr(out))
    return out


def attend_subset(q, hc: HeadCache, idx) -> np.ndarray:
    idx = np.ascontiguousarray(idx, np.int32)
    assert idx.size >= 1
    q = _f16bits(q).reshape(-1)
    out = np.zeros(hc.d, np.float64)
    lib().oracle_attend_subset(hc.d, idx.size, _ptr(idx), _ptr(q), *hc.kargs(), *hc.vargs(), _ptr(out))
    return out


def select_topk(s, k: int) -> np.ndarray:
    s = np.ascontiguousarray(s, np.float64)
    sel = np.zeros(k, np.int32)
    lib().oracle_select_topk(s.size, _ptr(s), k, _ptr(sel))
    return sel


def attend_topk(q, hc: HeadCache, k: int, T: int | None = None):
    """Top-k sparse decode attention; returns (out fp64 [d], sel int32 [k] ascending)."""
    T = hc.T if T is None else T
    assert 1 <= k <= T <= hc.T
    q = _f16bits(q).reshape(-1)
    out = np.zeros(hc.d, np.float64)
    sel = np.zeros(k, np.int32)
    lib().oracle_attend_topk(hc.d, T, k, _ptr(q), *hc.kargs(), *hc.vargs(), _ptr(out), _ptr(sel))
    return out, sel


def attend_rows(q, khat, vhat) -> np.ndarray:
    """Decode attention of one query over explicit dequantised rows khat, vhat [T][d]
    (float64); fp64 result [d]."""
    q = _f16bits(q).reshape(-1)
    khat = np.ascontiguousarray(khat, np.float64)
    vhat = np.ascontiguousarray(vhat, np.float64)
    T, d = khat.shape
    assert vhat.shape == (T, d) and q.size == d and T >= 1
    out = np.zeros(d, np.float64)
    lib().oracle_attend_rows(d, T, _ptr(q), _ptr(khat), _ptr(vhat), _ptr(out))
    return out


def attend_f16form(q, hc: HeadCache, T: int | None = None, idx=None) -> np.ndarray:
    """Attention over the cache in the report's FP16 form ("dequantised to FP16 before
    compute"): every dequantised K and V element rounded to binary16 (dequant_rows_f16),
    then the softmax and P.V of attend.  idx (optional): attend over those tokens only
    (the sparse variant on a given selection)."""
    T = hc.T if T is None else T
    rows = np.arange(T) if idx is None else np.ascontiguousarray(idx, np.int64)
    k16 = dequant_rows_f16(hc.kc[rows], hc.kmin[rows], hc.ksc[rows]).astype(np.float64)
    v16 = dequant_rows_f16(hc.vc[rows], hc.vmin[rows], hc.vsc[rows]).astype(np.float64)
    return attend_rows(q, k16, v16)


def prefill_attend(q, k, v) -> np.ndarray:
    """Causal prefill attention of one (batch row, head) over its prompt, fp16 inputs
    [s][d] (or [s][...][d] views with the head's rows strided, e.g. x[bi, :, ai]); fp64 [s][d]."""
    q, k, v = (_f16bits(np.asarray(x)) for x in (q, k, v))
    s, d = q.shape
    assert k.shape == (s, d) and v.shape == (s, d)
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    out = np.zeros((s, d), np.float64)
    lib().oracle_prefill_attend(d, s, d, _ptr(q), _ptr(k), _ptr(v), _ptr(out))
    return out


def prefill_attend_rows(q, k, v, rows) -> np.ndarray:
    """The causal prefill attention of one (batch row, head) at the query rows `rows` only
    (each 0..s-1); fp64 [len(rows)][d].  Same inputs as prefill_attend."""
    q, k, v = (_f16bits(np.asarray(x)) for x in (q, k, v))
    s, d = q.shape
    assert k.shape == (s, d) and v.shape == (s, d)
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    rows = np.ascontiguousarray(rows, np.int32)
    assert rows.ndim == 1 and np.all((rows >= 0) & (rows < s))
    out = np.zeros((rows.size, d), np.float64)
    lib().oracle_prefill_attend_rows(d, s, d, _ptr(q), _ptr(k), _ptr(v), rows.size, _ptr(rows), _ptr(out))
    return out


# ------------------------------------------------------------ int4 weights
def w_dequant(code: int, min16, scale16) -> np.float16:
    """FP16 form of one dequantised weight: binary16 nearest to min + code*scale."""
    mb = int(np.float16(min16).view(np.uint16))
    sb = int(np.float16(scale16).view(np.uint16))
    return np.uint16(lib().oracle_w_dequant(int(code), mb, sb)).view(np.float16)


def quantize_weight(w):
    """W fp16 [N][K] -> (codes uint8 [N][K/2], mins float16 [N][K/64], scales float16 [N][K/64])."""
    return quantize_rows_m16(w)


def gemm_w4a16(x, codes, mins, scales) -> np.ndarray:
    """y = x W^T (binary64) with W^ the FP16 form of the dequantised int4 weights.
    x fp16 [M][K]; codes [N][K/2]; mins/scales float16 [N][K/64]."""
    x = _f16bits(x)
    M, K = x.shape
    codes = np.ascontiguousarray(codes, np.uint8)
    N = codes.shape[0]
    assert codes.shape == (N, K // 2)
    mins = _f16bits(np.ascontiguousarray(mins, np.float16))
    scales = _f16bits(np.ascontiguousarray(scales, np.float16))
    assert mins.shape == (N, K // GROUP) and scales.shape == (N, K // GROUP)
    y = np.zeros((M, N), np.float64)
    lib().oracle_gemm_w4a16(M, N, K, _ptr(x), _ptr(codes), _ptr(mins), _ptr(scales), _ptr(y))
    return y
