"""GPU parity with binary16 min/scale planes (KVQ_META_F16) against the oracle's
binary16-metadata codec.

The same bar as with binary32 planes: codes, mins and scales bit-exact;
attention within 2e-3 + 1e-2 |oracle| element-wise.  The oracle dequantises
with the stored binary16 pair (widened exactly), so the attention reference
differs from the binary32 one only through the metadata.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_prefill_amd as kvq
import workloads as W
from tests.gpu_common import (HostCache, all_pairs, assert_close, f16_np, log, oracle_attend_pairs, require_gpu,
                              sample_pairs)
from tests.test_parity_gpu import (DEV, _check_prefill_full, _check_prefill_pairs, _gpu_rows, _nan_out, _small_cache,
                                   _topk_checks, run_decode_workload)

pytestmark = pytest.mark.gpu
META = "f16"


def test_m16_tiny_config_full():
    """b=2, a=2, d=64, s=16, n=4: every plane and every output, every step."""
    run_decode_workload(W.TINY, full_planes=True, attend_pairs_full_steps=range(1, 5), sample_n=4, meta=META)


@pytest.mark.timeout(600)
def test_m16_opt_6_7b_layer_full():
    """b=32, a=32, d=128, s=512 -> 544: planes in full, attention for all pairs at steps 1 and 32."""
    run_decode_workload(W.OPT_6_7B, full_planes=True, attend_pairs_full_steps=(1, 32), sample_n=64, meta=META)


@pytest.mark.timeout(600)
def test_m16_opt_30b_layer_sampled():
    """b=256, a=56, d=128 with 1% outlier channels x8: appended rows in full, sampled pairs."""
    run_decode_workload(W.OPT_30B, full_planes=False, attend_pairs_full_steps=(), sample_n=96, meta=META,
                        f16form=False)


@pytest.mark.timeout(600)
def test_m16_opt_175b_layer_sampled():
    """b=144, a=96, d=128, s=512 -> 544: appended rows in full, sampled pairs."""
    run_decode_workload(W.OPT_175B, full_planes=False, attend_pairs_full_steps=(), sample_n=96, meta=META)


@pytest.mark.timeout(600)
def test_m16_sparse_top10_layer_sampled():
    """b=32, a=96, context 2048 with boosted keys, keep 205, binary16 planes."""
    require_gpu()
    w = W.SPARSE
    T = w.s + w.n
    k_top = w.k_top(T)
    cache = kvq.QuantKVCache(w.b, w.a, w.h, w.s, w.n, device=DEV, fill=0xFF, meta=META)
    k, v = W.prefill_kv(w, 0, DEV)
    kvq.kv_quantize_prefill(cache, k, v)
    q, kn, vn = W.decode_inputs(w, 0, 1, DEV)
    kvq.kv_append_quant(cache, kn, vn, w.s)
    out, sel = kvq.decode_attention_q4_topk(cache, q, T, k_top, out=_nan_out(w.b, w.a, w.d))
    torch.cuda.synchronize()
    pairs = sample_pairs(w.b, w.a, 64, seed=56)
    hc = HostCache(w.b, w.a, w.d, w.S, META)
    hc.prefill(f16_np(k), f16_np(v), pairs)
    hc.append(f16_np(kn), f16_np(vn), w.s)
    _check_prefill_pairs(cache, hc, T, pairs, w.name + " m16")
    same = _topk_checks(hc, f16_np(q), T, k_top, pairs, _gpu_rows(out, pairs), sel.cpu().numpy(), w.name + " m16")
    log(f"[{w.name} m16] {len(pairs)} pairs ok; selection identical to the oracle's on {same}")
    assert same >= len(pairs) * 0.9


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("T", [1, 17, 65, 255, 543])
def test_m16_dense_ragged_contexts(d, T):
    require_gpu()
    b, a = 3, 5
    cache, hc, q = _small_cache(b, a, d, T, 3, 4000 + T + d, meta=META)
    pairs = all_pairs(b, a)
    out = kvq.decode_attention_q4(cache, q, T, out=_nan_out(b, a, d))
    torch.cuda.synchronize()
    ref = oracle_attend_pairs(hc, f16_np(q), T, pairs)
    assert_close(_gpu_rows(out, pairs), ref, f"m16 d={d} T={T}")


@pytest.mark.parametrize("splits", [1, 7])
@pytest.mark.parametrize("unroll,wpp", [(1, 1), (4, 2), (2, 4)])
def test_m16_dense_launch_shapes_and_splits(splits, unroll, wpp):
    require_gpu()
    b, a, d, T = 2, 3, 128, 700
    cache, hc, q = _small_cache(b, a, d, T, 0, 4200, meta=META)
    pairs = all_pairs(b, a)
    out = kvq.decode_attention_q4_tuned(cache, q, T, unroll, wpp, out=_nan_out(b, a, d), num_splits=splits)
    torch.cuda.synchronize()
    ref = oracle_attend_pairs(hc, f16_np(q), T, pairs)
    assert_close(_gpu_rows(out, pairs), ref, f"m16 splits={splits} unroll={unroll} wpp={wpp}")


def test_m16_codec_special_values():
    """Constant groups, signed zeros, fp16 extremes, subnormals, binary16 scales that are
    subnormal or underflow to 0, scales that round up or down: planes bit-exact."""
    require_gpu()
    b, a, d, s = 2, 4, 128, 48
    r = np.random.default_rng(79)
    x = r.standard_normal((b, s, a, d))
    x[0, 0] = 0.75                                   # constant rows
    x[0, 1] = 0.0
    x[0, 1, :, ::2] = -0.0                           # mixed-sign zeros
    x[0, 2] = np.where(r.random((a, d)) < 0.5, -65504.0, 65504.0)  # extremes
    x[0, 3] *= 1e-6                                  # fp16 subnormals
    x[0, 4, :, 0] = 60000.0                          # one huge element per row
    x[0, 5] = 0.0
    x[0, 5, :, 7] = 2.0 ** -24                       # range 2^-24: the binary16 scale underflows to 0
    x[0, 6] = 0.0
    x[0, 6, :, 3] = 2.0 ** -20                       # subnormal scale 2^-24: the top code clamps
    x[0, 6, :, 9] = 2.0 ** -21
    x[0, 7] = r.integers(0, 40, (a, d)) * 2.0 ** -24  # assorted subnormal scales
    x[0, 8] = 0.0
    x[0, 8, :, :4] = [0, 2000, 1800, 1000]            # scale rounds up to 133.375: codes 13 and 7
    x[1, :10] = np.round(x[1, :10] * 4) / 4          # many duplicates
    x[1, 10] = -x[1, 10] ** 2 * 100                  # negative-only groups
    x[1, 11:20] *= np.exp(r.uniform(-12, 9, (9, 1, 1)))  # scales across the binary16 range
    k = torch.from_numpy(x.astype(np.float16)).to(DEV)
    v = torch.from_numpy((-x).astype(np.float16)).to(DEV)
    cache = kvq.QuantKVCache(b, a, a * d, s, 0, device=DEV, fill=0xFF, meta=META)
    kvq.kv_quantize_prefill(cache, k, v)
    torch.cuda.synchronize()
    hc = HostCache(b, a, d, s, META)
    hc.prefill(f16_np(k), f16_np(v))
    _check_prefill_full(cache, hc, s, "m16 special values")
    assert float(hc.ksc[0, 0, 5, 0]) == 0.0 and float(hc.ksc[0, 0, 6, 0]) == 2.0 ** -24
    q = W.random_fp16((b, 1, a, d), 80, DEV)
    out = kvq.decode_attention_q4(cache, q, s)
    torch.cuda.synchronize()
    pairs = all_pairs(b, a)
    ref = oracle_attend_pairs(hc, f16_np(q), s, pairs)
    got = _gpu_rows(out, pairs).astype(np.float64)
    # With binary16 metadata the top level min + 15*scale of a group spanning the fp16
    # extremes is 65536 (scale 131008/15 rounds up to 8736), beyond the largest fp16 value.
    # Where the softmax puts its weight on such a row the exact output lies outside the fp16
    # range; there the output must be the fp16 rounding of the exact value (+-inf).
    big = np.abs(ref) > 65504
    with np.errstate(over="ignore"):
        assert np.array_equal(got[big], ref[big].astype(np.float16).astype(np.float64))
    log(f"m16 special values: {int(big.sum())} outputs beyond the fp16 range, rounded as fp16")
    assert_close(got[~big][None], ref[~big][None], "m16 special values attention")


@pytest.mark.parametrize("T", [1, 20, 64, 2048, 3000])
def test_m16_topk_small_and_long(T):
    """Top-k at k = 1, 10% and T over binary16 planes; both select kernels."""
    require_gpu()
    b, a, d = 2, 3, 128
    cache, hc, q = _small_cache(b, a, d, T, 0, 4300 + T, meta=META)
    pairs = all_pairs(b, a)
    for k_top in sorted({1, max(1, math.ceil(0.1 * T)), T}):
        out, sel = kvq.decode_attention_q4_topk(cache, q, T, k_top, out=_nan_out(b, a, d))
        torch.cuda.synchronize()
        _topk_checks(hc, f16_np(q), T, k_top, pairs, _gpu_rows(out, pairs), sel.cpu().numpy(),
                     f"m16 topk T={T} k={k_top}")


@pytest.mark.parametrize("d,b,a,s,pos,splits", [
    (128, 3, 5, 40, 40, 0), (128, 2, 3, 600, 640, 3), (64, 2, 2, 16, 16, 0), (256, 2, 3, 100, 150, 2),
])
def test_m16_fused_step_bit_identical_to_separate_calls(d, b, a, s, pos, splits):
    """kv_append_attend_q4 == kv_append_quant + decode_attention_q4 with binary16 planes."""
    require_gpu()
    n = max(1, pos - s + 1)
    S = s + n
    seed = 4400 + d + pos
    k = W.random_fp16((b, S, a, d), seed, DEV)
    v = W.random_fp16((b, S, a, d), seed + 1, DEV)
    kn = W.random_fp16((b, 1, a, d), seed + 2, DEV)
    vn = W.random_fp16((b, 1, a, d), seed + 3, DEV)
    q = W.random_fp16((b, 1, a, d), seed + 4, DEV)
    c1 = kvq.QuantKVCache(b, a, a * d, s, n, device=DEV, fill=0xFF, meta=META)
    c2 = kvq.QuantKVCache(b, a, a * d, s, n, device=DEV, fill=0xFF, meta=META)
    for c in (c1, c2):
        kvq.kv_quantize_prefill(c, k, v)
    kvq.kv_append_quant(c1, kn, vn, pos)
    o1 = kvq.decode_attention_q4(c1, q, pos + 1, out=_nan_out(b, a, d), num_splits=splits)
    o2 = kvq.kv_append_attend_q4(c2, q, kn, vn, pos, out=_nan_out(b, a, d), num_splits=splits)
    torch.cuda.synchronize()
    for t1, t2 in zip(c1.planes(), c2.planes()):
        assert torch.equal(t1.view(torch.uint8), t2.view(torch.uint8))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    hc = HostCache(b, a, d, S, META)
    hc.prefill(f16_np(k), f16_np(v))
    hc.append(f16_np(kn), f16_np(vn), pos)
    _check_prefill_full(c2, hc, S, f"m16 fused d={d} pos={pos}")
    pairs = all_pairs(b, a)
    ref = oracle_attend_pairs(hc, f16_np(q), pos + 1, pairs)
    assert_close(_gpu_rows(o2, pairs), ref, f"m16 fused d={d} pos={pos}")
