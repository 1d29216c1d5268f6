"""GPU check of the codec's two divisions for every range it can meet.

Every quantiser of the library stores scale = rng/15 and takes the codes with
an inverse scale ("FlexGen研究学术报告", section 三.2(C): group-wise asymmetric
4-bit, min/max affine code); the kernels compute both quotients without the
generic division sequence (a constant-divisor correction for rng/15, reciprocal
+ Newton + residual correction for the inverse).  A group range is the binary32
difference of two fp16 values, so it lies in [2^-24, 2 * 65504]; this test runs
the device code (kvq_codec_params) on every binary32 value in [2^-24, 2^17] and
compares scale and inverse bit for bit with the oracle's quotients, for
binary32 and binary16 metadata.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_prefill_amd as kvq
from tests.gpu_common import log, require_gpu

pytestmark = pytest.mark.gpu

LO = int(np.float32(2.0 ** -24).view(np.uint32))
HI = int(np.float32(2.0 ** 17).view(np.uint32))
CHUNK = 1 << 25


@pytest.mark.parametrize("meta", ["f32", "f16"])
def test_codec_divisions_every_range(meta):
    require_gpu()
    log(f"[codec] {meta}: {HI - LO + 1} binary32 ranges in [2^-24, 2^17]")
    bad = 0
    for start in range(LO, HI + 1, CHUNK):
        n = min(CHUNK, HI + 1 - start)
        bits = torch.arange(start, start + n, dtype=torch.int64, device="cuda").to(torch.int32)
        rng = bits.view(torch.float32)
        scale, inv = kvq.kvq_codec_params(rng, meta)
        r_np = (np.arange(start, start + n, dtype=np.uint64).astype(np.uint32)).view(np.float32)
        want_s, want_i = oracle.codec_params(r_np, meta)
        got_s = scale.cpu().numpy()
        got_i = inv.cpu().numpy()
        ms = got_s.view(np.uint32) != want_s.view(np.uint32)
        mi = got_i.view(np.uint32) != want_i.view(np.uint32)
        if ms.any() or mi.any():
            k = int(np.flatnonzero(ms | mi)[0])
            log(f"[codec] first mismatch rng={r_np[k]!r}: scale {got_s[k]!r} vs {want_s[k]!r}, "
                f"inv {got_i[k]!r} vs {want_i[k]!r}")
        bad += int(ms.sum()) + int(mi.sum())
    assert bad == 0

