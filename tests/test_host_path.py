"""Parity of the host (CPU) path against the oracle -- runs without a GPU.

The host calls keep the cache in CPU memory and run the codec and the decode
attention on the CPU (the report's CPU delegation of attention).  Same bar as
the GPU path: codes, mins and scales bit-exact with the oracle's codec
(binary32 and binary16 metadata); attention within 2e-3 + 1e-2 |oracle|
element-wise, for the AVX-512 loop and for the scalar loop.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_prefill_amd as kvq
from tests.gpu_common import assert_close, oracle_planes_from_prompt

THREADS = 4


def _f16(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float16))


def _oracle_planes(x: np.ndarray, meta: str):
    """[b][s][a][d] fp16 -> oracle planes in cache order [b][a][s][...]."""
    return oracle_planes_from_prompt(x.view(np.uint16), meta)


def _check_planes(cache, kx, vx, s, meta, what):
    for name, x, gc, gm, gs in (("k", kx, cache.k_codes, cache.k_min, cache.k_scale),
                                ("v", vx, cache.v_codes, cache.v_min, cache.v_scale)):
        c, m, sc = _oracle_planes(x, meta)
        assert np.array_equal(gc[:, :, :s].numpy(), c), f"{what}: {name} codes"
        mt = np.uint16 if meta == "f16" else np.uint32
        assert np.array_equal(gm[:, :, :s].numpy().view(mt), m.view(mt)), f"{what}: {name} mins"
        assert np.array_equal(gs[:, :, :s].numpy().view(mt), sc.view(mt)), f"{what}: {name} scales"


def _special(r, b, s, a, d):
    x = r.standard_normal((b, s, a, d))
    x[0, 0] = 0.75                                   # constant rows
    x[0, 1] = 0.0
    x[0, 1, :, ::2] = -0.0                           # mixed-sign zeros
    x[0, 2] = np.where(r.random((a, d)) < 0.5, -65504.0, 65504.0)
    x[0, 3] *= 1e-6                                  # subnormals
    x[0, 4] = 0.0
    x[0, 4, :, 7] = 2.0 ** -24                       # binary16 scale underflows
    x[0, 5] = 0.0
    x[0, 5, :, :4] = [0, 2000, 1800, 1000]           # binary16 scale rounds up
    x[-1, -1] = np.round(x[-1, -1] * 4) / 4          # ties
    return x.astype(np.float16)


@pytest.mark.parametrize("meta", ["f32", "f16"])
@pytest.mark.parametrize("simd", [True, False])
@pytest.mark.parametrize("d", [64, 256])
def test_host_codec_bit_exact(meta, simd, d):
    """Prefill and append planes equal the oracle's codec bit for bit (AVX-512 and scalar
    codec), with constant, zero, extreme, subnormal and tie groups."""
    r = np.random.default_rng(6000 + d)
    b, a, s, n = 2, 3, 24, 4
    k, v = _special(r, b, s, a, d), _special(r, b, s, a, d)
    cache = kvq.QuantKVCache(b, a, a * d, s, n, device="cpu", fill=0xFF, meta=meta)
    kvq.kvq_host_use_simd(simd)
    try:
        kvq.kv_quantize_prefill_host(cache, _f16(k), _f16(v), n_threads=THREADS)
        _check_planes(cache, k, v, s, meta, f"prefill meta={meta} simd={simd}")
        kn = r.standard_normal((b, 1, a, d)).astype(np.float16)
        vn = r.standard_normal((b, 1, a, d)).astype(np.float16)
        kvq.kv_append_quant_host(cache, _f16(kn), _f16(vn), s, n_threads=THREADS)
    finally:
        kvq.kvq_host_use_simd(True)
    _check_planes(cache, np.concatenate([k, kn], 1), np.concatenate([v, vn], 1), s + 1, meta,
                  f"append meta={meta} simd={simd}")


def test_host_codec_random_scales_bit_exact():
    """Many groups with scales across the binary16 range (both metadata types): the AVX-512
    codec against the oracle."""
    r = np.random.default_rng(6050)
    b, a, d, s = 4, 8, 128, 64
    x = r.standard_normal((b, s, a, d)) * np.exp(r.uniform(-14, 10, (b, s, a, 1)))
    x = np.clip(x, -65504, 65504).astype(np.float16)
    for meta in ("f32", "f16"):
        cache = kvq.QuantKVCache(b, a, a * d, s, 0, device="cpu", fill=0xFF, meta=meta)
        kvq.kv_quantize_prefill_host(cache, _f16(x), _f16(-x), n_threads=THREADS)
        _check_planes(cache, x, -x, s, meta, f"random scales meta={meta}")


def _attend_case(b, a, d, T, seed, meta="f32", simd=True, std=1.0, ramp=False):
    r = np.random.default_rng(seed)
    k = r.standard_normal((b, T, a, d)) * std
    if ramp:
        k = k * 0.1 + np.linspace(0.0, 6.0, T)[None, :, None, None]
    k = k.astype(np.float16)
    v = (r.standard_normal((b, T, a, d)) * std).astype(np.float16)
    q = (r.standard_normal((b, 1, a, d)) * std).astype(np.float16)
    cache = kvq.QuantKVCache(b, a, a * d, T, 1, device="cpu", fill=0xFF, meta=meta)
    kvq.kv_quantize_prefill_host(cache, _f16(k), _f16(v), n_threads=THREADS)
    kvq.kvq_host_use_simd(simd)
    try:
        out = kvq.decode_attention_q4_host(cache, _f16(q), T, n_threads=THREADS)
    finally:
        kvq.kvq_host_use_simd(True)
    kc, km, ks = _oracle_planes(k, meta)
    vc, vm, vs = _oracle_planes(v, meta)
    qb = q.view(np.uint16)
    ref = np.stack([oracle.attend(np.ascontiguousarray(qb[bi, 0, ai]),
                                  oracle.HeadCache(kc[bi, ai], km[bi, ai], ks[bi, ai], vc[bi, ai], vm[bi, ai],
                                                   vs[bi, ai]), T)
                    for bi in range(b) for ai in range(a)])
    got = out.float().numpy()[:, 0].reshape(b * a, d)
    return assert_close(got, ref, f"host b={b} a={a} d={d} T={T} meta={meta} simd={simd}")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("T", [1, 2, 17, 65, 300])
def test_host_attention_ragged(d, T):
    _attend_case(2, 3, d, T, 6100 + d + T)


@pytest.mark.parametrize("meta", ["f32", "f16"])
@pytest.mark.parametrize("simd", [True, False])
def test_host_attention_paths_and_metadata(meta, simd):
    """The AVX-512 loop and the scalar loop, binary32 and binary16 metadata."""
    _attend_case(2, 4, 128, 200, 6200, meta=meta, simd=simd)


@pytest.mark.parametrize("simd", [True, False])
def test_host_attention_rising_scores(simd):
    """Keys shifted by a ramp along the context, so each head's scores drift steadily up
    (or down, with the sign of sum(q)): where they rise the running max moves in every
    block and the accumulators are rescaled each time."""
    _attend_case(2, 2, 128, 333, 6250, simd=simd, ramp=True)


def test_host_attention_opt_layer_sample():
    """An OPT-shaped slice (8 batch rows x 32 heads, d = 128, context 544) with the
    OPT-30B-style magnitude (std 4)."""
    _attend_case(8, 32, 128, 544, 6300, std=4.0)


def test_host_matches_errors():
    cache = kvq.QuantKVCache(1, 2, 256, 8, 2, device="cpu")
    q = _f16(np.zeros((1, 1, 2, 128)))
    with pytest.raises(kvq.KvqError):
        kvq.decode_attention_q4_host(cache, q, 11)
    with pytest.raises(kvq.KvqError):
        kvq.kv_append_quant_host(cache, q, q, 10)
    with pytest.raises(TypeError):
        kvq.decode_attention_q4_host(cache, q.float(), 4)
