"""GPU parity of the int4-weight decode projections against the oracle.

kvq_w4_quantize: codes, mins and scales bit-exact with the oracle's
binary16-metadata codec.  gemm_w4a16: y = x W^T against the oracle's binary64
product with the FP16-form weights, element-wise within a bound derived from
the arithmetic: the fp16 output rounding (2^-11 |y|) plus binary32
accumulation over the K/32 matrix-core steps of a chain (and the split sum),
(K/32 + 8) * 2^-24 * sum_k |x_k w_k|, plus the fp16 subnormal spacing.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_prefill_amd as kvq
import workloads as W
from tests.gpu_common import assert_bits_equal, log, require_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def tile_planes(codes, mins, scales):
    """Oracle planes [N][K/2], [N][K/64] rearranged into the device's tiled layout
    (a reindexing only): codes [N/64][K/128][64][64], mins/scales [N/64][K/128][64][2]."""
    N, K2 = codes.shape
    ct = codes.reshape(N // 64, 64, K2 // 64, 64).transpose(0, 2, 1, 3)
    mt = mins.reshape(N // 64, 64, K2 // 64, 2).transpose(0, 2, 1, 3)
    st = scales.reshape(N // 64, 64, K2 // 64, 2).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(ct), np.ascontiguousarray(mt), np.ascontiguousarray(st)


def _unpack(codes):
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], -1).astype(np.float64)


def _w_hat(codes, mins, scales):
    """FP16-form weights (numpy's binary16 rounding of min + c*scale in binary64; pinned
    equal to the oracle's dequant)."""
    c = _unpack(codes)
    g = np.repeat(np.arange(c.shape[1] // 64), 64)
    return (mins.astype(np.float64)[:, g] + c * scales.astype(np.float64)[:, g]).astype(np.float16)


def assert_gemm_close(y_gpu: np.ndarray, y_ref: np.ndarray, mag: np.ndarray, K: int, what: str):
    bound = 2.0 ** -11 * np.abs(y_ref) + (K / 32 + 8) * 2.0 ** -24 * mag + 2.0 ** -24
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, (f"{what}: {len(bad)} outputs out of bound, first {bad[:3].tolist()}, "
                           f"err {err[tuple(bad[0])]:.3g} bound {bound[tuple(bad[0])]:.3g}")
    rel = float((err / np.maximum(mag, 1e-30)).max())
    return rel


def _weights(N, K, seed, std=0.02, special=False):
    w = W.random_fp16((N, K), seed, DEV, std)
    if special:
        wn = w.cpu().numpy()
        wn[0] = 0.0                                 # zero rows: scale 0
        wn[1] = np.float16(0.75)                    # constant groups
        wn[2, ::2] = -0.0                           # mixed-sign zeros
        wn[3] = np.where(np.arange(K) % 2, 65504.0, -65504.0)  # extremes: dequantised top level overflows
        wn[4] *= np.float16(1e-4)                   # subnormal scales
        wn[5, :64] = 0.0
        wn[5, 7] = 2.0 ** -24                       # scale underflows to 0
        w = torch.from_numpy(wn).to(DEV)
    return w


def _run(M, N, K, seed, splits=0, std=0.02, xstd=1.0, special=False):
    """GPU: quantise W and form y.  Oracle: its own planes from the same fp16 W, checked
    equal to the GPU's (tiled), and its product from them."""
    w = _weights(N, K, seed, std, special)
    x = W.random_fp16((M, K), seed + 1, DEV, xstd)
    codes, mins, scales = kvq.kvq_w4_quantize(w)
    y = kvq.gemm_w4a16(x, codes, mins, scales, num_splits=splits)
    torch.cuda.synchronize()
    c, m, s = oracle.quantize_weight(w.cpu().numpy())
    ct, mt, st = tile_planes(c, m, s)
    assert_bits_equal(codes, ct, "w codes")
    assert_bits_equal(mins, mt, "w mins")
    assert_bits_equal(scales, st, "w scales")
    return x, (codes, mins, scales), (c, m, s), y


def test_w4_quantize_bit_exact():
    """Weight planes equal the oracle's binary16-metadata codec bit for bit, including zero,
    constant, extreme, subnormal and underflowing groups."""
    require_gpu()
    N, K = 320, 640
    w = _weights(N, K, 5000, special=True)
    codes, mins, scales = kvq.kvq_w4_quantize(w)
    torch.cuda.synchronize()
    ct, mt, st = tile_planes(*oracle.quantize_weight(w.cpu().numpy()))
    assert_bits_equal(codes, ct, "w codes")
    assert_bits_equal(mins, mt, "w mins")
    assert_bits_equal(scales, st, "w scales")


@pytest.mark.parametrize("M", [1, 7, 16, 33, 144, 150])
@pytest.mark.parametrize("N,K", [(64, 128), (320, 640), (256, 1024)])
@pytest.mark.parametrize("splits", [0, 1, 3, kvq.KVQ_GEMM_STREAM])
def test_gemm_shapes_full(M, N, K, splits):
    """Every output of small shapes: row tiles with ragged ends (M not a multiple of 16 or
    of 144), partial column groups (N = 64, 320), K ranges split 1, 3 ways, automatically or
    in the stream form."""
    require_gpu()
    if splits > K // 128:
        # more splits than 128-wide chunks of K: refused on the host, nothing enqueued
        w = _weights(N, K, 5100 + M + N + K + splits)
        x = W.random_fp16((M, K), 5101 + M + N + K + splits, DEV)
        codes, mins, scales = kvq.kvq_w4_quantize(w)
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        with pytest.raises(kvq.KvqError) as ei:
            kvq.gemm_w4a16(x, codes, mins, scales, y=y, num_splits=splits)
        assert ei.value.status == -2
        assert kvq.kvq_gemm_w4_workspace_bytes(M, N, K, splits) == 0
        torch.cuda.synchronize()
        assert torch.isnan(y.float()).all()
        return
    x, _, (c, m, s), y = _run(M, N, K, 5100 + M + N + K + splits)
    xh = x.cpu().numpy()
    ref = oracle.gemm_w4a16(xh, c, m, s)
    mag = np.abs(xh.astype(np.float64)) @ np.abs(_w_hat(c, m, s).astype(np.float64)).T
    rel = assert_gemm_close(y.float().cpu().numpy(), ref, mag, K, f"M={M} N={N} K={K} splits={splits}")
    log(f"gemm M={M} N={N} K={K} splits={splits}: max err / sum|x w| = {rel:.2e}")


def test_gemm_special_weights_and_large_inputs():
    """Zero, constant, subnormal-scale weight rows and inputs of large magnitude.  The
    row spanning the fp16 extremes dequantises beyond 65504 (the binary16 scale rounds
    up): its outputs are checked only where the exact result is finite in fp16."""
    require_gpu()
    M, N, K = 40, 128, 512
    x, _, (c, m, s), y = _run(M, N, K, 5200, xstd=30.0, special=True)
    xh = x.cpu().numpy()
    ref = oracle.gemm_w4a16(xh, c, m, s)
    with np.errstate(over="ignore", invalid="ignore"):
        wh = np.abs(_w_hat(c, m, s).astype(np.float64))
        mag = np.abs(xh.astype(np.float64)) @ np.where(np.isfinite(wh), wh, 0.0).T
    ok = np.all(np.isfinite(_w_hat(c, m, s)), axis=1)       # weight rows without an overflowing level
    yg = y.float().cpu().numpy()
    assert_gemm_close(yg[:, ok], ref[:, ok], mag[:, ok], K, "special weights")
    assert np.all(yg[:, 0] == 0.0)                           # zero row


@pytest.mark.timeout(300)
@pytest.mark.parametrize("N", [12288, 36864])
def test_gemm_opt175b_projection_sampled(N):
    """The OPT-175B decode projections (M = 144, K = 12288; N = 12288 output, split form;
    N = 36864 fused QKV, stream form) in the launch configuration the benchmark times:
    three sampled 64-row weight tiles (first, last, one seeded) bit-exact, their output
    columns for all 144 rows within the bound."""
    require_gpu()
    M, K = 144, 12288
    log(f"[gemm] M={M} N={N} K={K}: quantise + product")
    w = _weights(N, K, 5300 + (N != K))
    x = W.random_fp16((M, K), 5301, DEV)
    codes, mins, scales = kvq.kvq_w4_quantize(w)
    y = kvq.gemm_w4a16(x, codes, mins, scales)
    torch.cuda.synchronize()
    # sampled 64-row tiles: the oracle quantises those rows of W and checks the GPU's tiles
    tiles = np.sort(np.random.default_rng(53).choice(N // 64, 3, replace=False))
    tiles[0], tiles[-1] = 0, N // 64 - 1
    rows = np.concatenate([np.arange(64 * t, 64 * t + 64) for t in tiles])
    wh = w.cpu().numpy()[rows]
    c, m, s = oracle.quantize_weight(wh)
    ct, mt, st = tile_planes(c, m, s)
    tix = torch.from_numpy(tiles).to(DEV)
    assert_bits_equal(codes[tix], ct, "w codes (sampled tiles)")
    assert_bits_equal(mins[tix], mt, "w mins (sampled tiles)")
    assert_bits_equal(scales[tix], st, "w scales (sampled tiles)")
    xh = x.cpu().numpy()
    ref = oracle.gemm_w4a16(xh, c, m, s)
    mag = np.abs(xh.astype(np.float64)) @ np.abs(_w_hat(c, m, s).astype(np.float64)).T
    rel = assert_gemm_close(y.float().cpu().numpy()[:, rows], ref, mag, K, "OPT-175B projection")
    log(f"[gemm] OPT-175B projection N={N}: {len(rows)} columns x 144 rows ok, max err / sum|x w| = {rel:.2e}")


# (M, N, K): stream-form cuts.  33 x 1280 x 384: 5 tiles of 3 chunks over 3 workgroups of 5
# units -- whole tiles in the middle of a range, a tile's head and tail in different
# workgroups; 150 x 1536 x 1920: 90 units over 22 workgroups, every tile cut 4 or 5 ways at
# ragged places; 161 x 768 x 1152: two row tiles (the second 1 row) of 9 chunks over 13
# workgroups; 16 x 64 x 2048: one tile cut 4 ways.
@pytest.mark.parametrize("M,N,K", [(33, 1280, 384), (150, 1536, 1920), (161, 768, 1152), (16, 64, 2048)])
def test_gemm_stream_form_cuts(M, N, K):
    """Every output of the stream form where its ranges cut tiles in every way."""
    require_gpu()
    x, _, (c, m, s), y = _run(M, N, K, 5500 + M + N + K, splits=kvq.KVQ_GEMM_STREAM)
    xh = x.cpu().numpy()
    ref = oracle.gemm_w4a16(xh, c, m, s)
    mag = np.abs(xh.astype(np.float64)) @ np.abs(_w_hat(c, m, s).astype(np.float64)).T
    rel = assert_gemm_close(y.float().cpu().numpy(), ref, mag, K, f"stream M={M} N={N} K={K}")
    log(f"gemm stream M={M} N={N} K={K}: max err / sum|x w| = {rel:.2e}")


def test_gemm_deterministic_and_split_invariant():
    """Two runs are bit-identical; split counts and the stream form agree to binary32
    rounding."""
    require_gpu()
    M, N, K = 144, 512, 2048
    x, (codes, mins, scales), _, y1 = _run(M, N, K, 5400)
    y2 = kvq.gemm_w4a16(x, codes, mins, scales)
    y3 = kvq.gemm_w4a16(x, codes, mins, scales, num_splits=1)
    y4 = kvq.gemm_w4a16(x, codes, mins, scales, num_splits=16)
    y5 = kvq.gemm_w4a16(x, codes, mins, scales, num_splits=kvq.KVQ_GEMM_STREAM)
    y6 = kvq.gemm_w4a16(x, codes, mins, scales, num_splits=kvq.KVQ_GEMM_STREAM)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y5.view(torch.int16), y6.view(torch.int16))
    a, b, d, e = y3.float(), y4.float(), y1.float(), y5.float()
    assert float((a - b).abs().max()) <= float(2.0 ** -9 * a.abs().max() + 1e-3)
    assert float((a - d).abs().max()) <= float(2.0 ** -9 * a.abs().max() + 1e-3)
    assert float((a - e).abs().max()) <= float(2.0 ** -9 * a.abs().max() + 1e-3)
