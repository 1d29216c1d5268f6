"""Helpers shared by the GPU parity tests: move tensors to the oracle, compare.

The oracle only ever receives the fp16 inputs (copied to the host) and its own
quantised planes; nothing produced by the HIP path is fed back into it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np
import torch

import oracle

ATOL = 2e-3
RTOL = 1e-2


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU (run with -m 'not gpu' on CPU)"


def f16_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint16)


QUANTIZE = {"f32": oracle.quantize_rows, "f16": oracle.quantize_rows_m16}
META_NP = {"f32": np.float32, "f16": np.float16}


def oracle_planes_from_prompt(k: np.ndarray, meta: str = "f32") -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Prompt rows [b][s][a][d] (fp16 bits) -> oracle planes in cache order [b][a][s][...]."""
    codes, mins, scales = QUANTIZE[meta](k)
    return (np.ascontiguousarray(codes.transpose(0, 2, 1, 3)), np.ascontiguousarray(mins.transpose(0, 2, 1, 3)),
            np.ascontiguousarray(scales.transpose(0, 2, 1, 3)))


def oracle_row(x: np.ndarray, meta: str = "f32"):
    """New-token rows [b][1][a][d] -> oracle planes [b][a][...] of that slot."""
    codes, mins, scales = QUANTIZE[meta](x[:, 0])
    return codes, mins, scales


def assert_bits_equal(gpu: torch.Tensor, ref: np.ndarray, what: str):
    g = gpu.detach().cpu().contiguous().numpy()
    if g.dtype == np.float32:
        g = g.view(np.uint32)
        assert np.asarray(ref).dtype == np.float32, (what, np.asarray(ref).dtype)
        ref = np.ascontiguousarray(ref, np.float32).view(np.uint32)
    elif g.dtype == np.float16:
        g = g.view(np.uint16)
        assert np.asarray(ref).dtype == np.float16, (what, np.asarray(ref).dtype)
        ref = np.ascontiguousarray(ref, np.float16).view(np.uint16)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    bad = np.argwhere(g != ref)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:3].tolist()}: gpu {g[tuple(bad[0])]} ref {ref[tuple(bad[0])]}"


class HostCache:
    """The oracle's own copy of a layer's planes, [b][a][S][...], filled from inputs.
    meta = "f32" or "f16": the metadata type, quantised by the matching oracle codec."""

    def __init__(self, b, a, d, S, meta: str = "f32"):
        G = d // 64
        self.meta = meta
        mt = META_NP[meta]
        self.kc = np.zeros((b, a, S, d // 2), np.uint8)
        self.vc = np.zeros((b, a, S, d // 2), np.uint8)
        self.kmin = np.zeros((b, a, S, G), mt)
        self.ksc = np.zeros((b, a, S, G), mt)
        self.vmin = np.zeros((b, a, S, G), mt)
        self.vsc = np.zeros((b, a, S, G), mt)

    def prefill(self, k: np.ndarray, v: np.ndarray, pairs=None):
        """k, v: [b][s][a][d] fp16 bits.  pairs: optional list of (bi, ai) to quantise only.
        Without pairs every batch row is quantised, batch rows spread over a thread pool."""
        s = k.shape[1]
        if pairs is None:
            def one(bi):
                kc, km, ks = oracle_planes_from_prompt(k[bi:bi + 1], self.meta)
                vc, vm, vs = oracle_planes_from_prompt(v[bi:bi + 1], self.meta)
                self.kc[bi, :, :s], self.kmin[bi, :, :s], self.ksc[bi, :, :s] = kc[0], km[0], ks[0]
                self.vc[bi, :, :s], self.vmin[bi, :, :s], self.vsc[bi, :, :s] = vc[0], vm[0], vs[0]
            with _pool() as ex:
                list(ex.map(one, range(k.shape[0])))
        else:
            for bi, ai in pairs:
                c, m, sc = QUANTIZE[self.meta](np.ascontiguousarray(k[bi, :, ai]))
                self.kc[bi, ai, :s], self.kmin[bi, ai, :s], self.ksc[bi, ai, :s] = c, m, sc
                c, m, sc = QUANTIZE[self.meta](np.ascontiguousarray(v[bi, :, ai]))
                self.vc[bi, ai, :s], self.vmin[bi, ai, :s], self.vsc[bi, ai, :s] = c, m, sc

    def append(self, k_new: np.ndarray, v_new: np.ndarray, pos: int):
        c, m, s = oracle_row(k_new, self.meta)
        self.kc[:, :, pos], self.kmin[:, :, pos], self.ksc[:, :, pos] = c, m, s
        c, m, s = oracle_row(v_new, self.meta)
        self.vc[:, :, pos], self.vmin[:, :, pos], self.vsc[:, :, pos] = c, m, s

    def head(self, bi, ai, T):
        return oracle.HeadCache(self.kc[bi, ai, :T], self.kmin[bi, ai, :T], self.ksc[bi, ai, :T], self.vc[bi, ai, :T],
                                self.vmin[bi, ai, :T], self.vsc[bi, ai, :T])


def _pool():
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    return cf.ThreadPoolExecutor(n)


def oracle_attend_pairs(hc: HostCache, q: np.ndarray, T: int, pairs) -> np.ndarray:
    """Dense oracle output for the given (bi, ai) pairs; q [b][1][a][d] fp16 bits."""
    with _pool() as ex:
        outs = list(ex.map(lambda p: oracle.attend(np.ascontiguousarray(q[p[0], 0, p[1]]), hc.head(p[0], p[1], T), T),
                           pairs))
    return np.stack(outs)


def oracle_attend_pairs_f16form(hc: HostCache, q: np.ndarray, T: int, pairs) -> np.ndarray:
    """The same pairs against attention over the FP16 form of the dequantised cache (every
    dequantised element rounded to binary16 before compute, as the report writes it)."""
    with _pool() as ex:
        outs = list(ex.map(lambda p: oracle.attend_f16form(np.ascontiguousarray(q[p[0], 0, p[1]]),
                                                           hc.head(p[0], p[1], T), T), pairs))
    return np.stack(outs)


def tolerance_ratio(gpu_rows: np.ndarray, ref_rows: np.ndarray) -> float:
    """max |gpu - ref| / (ATOL + RTOL |ref|): <= 1 is inside the bar."""
    return float(np.max(np.abs(gpu_rows.astype(np.float64) - ref_rows) / (ATOL + RTOL * np.abs(ref_rows))))


def assert_close(gpu_rows: np.ndarray, ref_rows: np.ndarray, what: str):
    """|gpu - ref| <= ATOL + RTOL*|ref| element-wise (ref = fp64 oracle)."""
    g = gpu_rows.astype(np.float64)
    err = np.abs(g - ref_rows)
    lim = ATOL + RTOL * np.abs(ref_rows)
    bad = np.argwhere(~(err <= lim))
    maxabs = float(err.max()) if err.size else 0.0
    assert bad.size == 0, (f"{what}: {len(bad)} elements out of tolerance, max abs err {maxabs:.3g}, "
                           f"first {bad[:3].tolist()}")
    return maxabs


def all_pairs(b, a):
    return [(bi, ai) for bi in range(b) for ai in range(a)]


def sample_pairs(b, a, n, seed):
    r = np.random.default_rng(seed)
    idx = r.choice(b * a, size=min(n, b * a), replace=False)
    ps = {(0, 0), (b - 1, a - 1)} | {(int(i) // a, int(i) % a) for i in idx}
    return sorted(ps)
