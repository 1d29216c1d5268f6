"""Evidence for one reading of the pages (CPU only).

"FlexGen研究学术报告" section 三.2(C) says the quantised KV cache is
dequantised to FP16 before compute.  The oracle's attention uses the exact
dequantised value min + code*scale instead, and keeps the FP16 form as a
reference function.  These tests record why: on ordinary N(0,1) inputs the
two agree far inside the 2e-3 + 1e-2|ref| tolerance, but with the OPT-30B
workload's x8 outlier channels in q and k the FP16 rounding of a
dequantised key moves a logit enough to exceed that tolerance, so an
FP16-rounded reference would measure rounding noise, not the method.
"""
import numpy as np

import oracle
from tests.oracle_pins import _sdpa


def _case(seed, T, d, outliers):
    r = np.random.default_rng(seed)
    K, V, q = r.standard_normal((T, d)), r.standard_normal((T, d)), r.standard_normal(d)
    if outliers:
        ch = r.choice(d, 2, replace=False)
        K[:, ch] *= 8
        V[:, ch] *= 8
        q[ch] *= 8
    K, V, q = K.astype(np.float16), V.astype(np.float16), q.astype(np.float16)
    kc, km, ks = oracle.quantize_rows(K)
    vc, vm, vs = oracle.quantize_rows(V)
    exact = oracle.attend(q, oracle.HeadCache(kc, km, ks, vc, vm, vs))
    k16 = oracle.dequant_rows_f16(kc, km, ks).astype(np.float64)
    v16 = oracle.dequant_rows_f16(vc, vm, vs).astype(np.float64)
    fp16_form = _sdpa(q.astype(np.float64), k16, v16)
    return np.max(np.abs(fp16_form - exact) / (2e-3 + 1e-2 * np.abs(exact)))


def test_fp16_form_is_inside_tolerance_on_plain_inputs():
    assert max(_case(s, 64, 128, False) for s in range(20)) < 0.5


def test_fp16_form_exceeds_tolerance_with_outlier_channels():
    assert _case(140, 4, 128, True) > 1.5
