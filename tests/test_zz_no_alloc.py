"""decode_attention_q4_noalloc: the allocation-free variant of decode_attention_q4, called
through the C ABI, against the allocating entry point and the oracle."""
from __future__ import annotations

import pytest
import torch

import quantized_kv_cache_prefill_amd as kvq
from tests.gpu_common import all_pairs, assert_close, f16_np, log, oracle_attend_pairs, require_gpu
from tests.test_parity_gpu import _gpu_rows, _nan_out, _small_cache

pytestmark = pytest.mark.gpu


def _one_call(b, a, d, T, num_splits, seed):
    cache, hc, q = _small_cache(b, a, d, T, 0, seed)
    need = kvq.kvq_workspace_bytes(cache, T, num_splits, 0)
    ref = kvq.decode_attention_q4(cache, q, T, out=_nan_out(b, a, d), num_splits=num_splits)
    torch.cuda.synchronize()
    out = _nan_out(b, a, d)
    before = torch.cuda.memory_allocated()
    kvq.decode_attention_q4_noalloc(cache, q, T, out, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "differs from decode_attention_q4"
    pairs = all_pairs(b, a)
    err = assert_close(_gpu_rows(out, pairs), oracle_attend_pairs(hc, f16_np(q), T, pairs),
                       f"noalloc b={b} a={a} d={d} T={T} splits={num_splits}")
    log(f"noalloc b={b} a={a} d={d} T={T} splits={num_splits}: {need} workspace bytes, max abs err {err:.2e}")
    return need


def test_noalloc_two_calls_second_smaller():
    """Two calls in a row, the second with a smaller input (fewer pairs, shorter context,
    other head_dim, explicit split count): each equals decode_attention_q4 bit for bit and the
    oracle within the bar; both use the static workspace (split partials)."""
    require_gpu()
    n1 = _one_call(2, 8, 128, 5000, 0, 8100)
    n2 = _one_call(1, 3, 64, 1300, 5, 8101)
    assert n1 > n2 > 0


def test_noalloc_without_splits_and_limit():
    """One split needs no workspace; a launch whose partials exceed the static workspace is
    refused with KVQ_ENOSPACE before anything is enqueued (the output keeps its fill)."""
    require_gpu()
    assert _one_call(2, 4, 128, 300, 1, 8102) == 0
    b, a, d, T = 64, 32, 256, 8192
    cache = kvq.QuantKVCache(b, a, a * d, T, 0, device="cuda", fill=0)
    assert kvq.kvq_workspace_bytes(cache, T, 256, 0) > kvq.KVQ_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((b, 1, a, d), dtype=torch.float16, device="cuda")
    out = _nan_out(b, a, d)
    with pytest.raises(kvq.KvqError) as ei:
        kvq.decode_attention_q4_noalloc(cache, q, T, out, num_splits=256)
    assert ei.value.status == -4
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
