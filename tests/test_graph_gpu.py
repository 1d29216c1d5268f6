"""HIP graph capture of the decode-step calls.  The library's entry points enqueue kernels
only -- no allocation, memset or synchronisation inside the library -- so one decode step
(append, then attention; the fused step; sparse attention; the allocation-free attention)
can be captured once and replayed.  Every replay is checked against the same calls made
eagerly on the same inputs, with eager work and synchronisations between the replays, and
one replay against the oracle."""
from __future__ import annotations

import pytest
import torch

import quantized_kv_cache_prefill_amd as kvq
import workloads as W
from tests.gpu_common import all_pairs, assert_close, f16_np, log, oracle_attend_pairs, require_gpu
from tests.test_parity_gpu import _gpu_rows, _small_cache

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16)


@pytest.mark.parametrize("num_splits", [1, 4])
def test_graph_append_then_attend(num_splits):
    """kv_append_quant at slot s, then decode_attention_q4 over s + 1 tokens (one split, or
    four with the workspace holding the split partials and the merge pass), captured."""
    require_gpu()
    b, a, d, s, n = 2, 3, 128, 300, 8
    cache, hc, q0 = _small_cache(b, a, d, s, n, 9300)
    T = s + 1
    kn = W.random_fp16((b, 1, a, d), 9301, DEV)
    vn = W.random_fp16((b, 1, a, d), 9302, DEV)
    q = q0.clone()
    out = torch.empty_like(q)
    need = kvq.kvq_workspace_bytes(cache, T, num_splits, 0)
    assert (need > 0) == (num_splits > 1)
    ws = torch.empty(max(need // 4, 4), dtype=torch.float32, device=DEV)
    kvq.kv_append_quant(cache, kn, vn, s)          # every kernel runs once before the capture
    kvq.decode_attention_q4(cache, q, T, out=out, num_splits=num_splits, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvq.kv_append_quant(cache, kn, vn, s)
        kvq.decode_attention_q4(cache, q, T, out=out, num_splits=num_splits, ws=ws)
    hc.append(f16_np(kn), f16_np(vn), s)
    for i in range(5):
        q.copy_(W.random_fp16((b, 1, a, d), 9310 + i, DEV))  # eager work between replays
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = kvq.decode_attention_q4(cache, q, T, num_splits=num_splits)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), f"replay {i} differs from the eager call"
        if i == 4:
            pairs = all_pairs(b, a)
            err = assert_close(_gpu_rows(out, pairs), oracle_attend_pairs(hc, f16_np(q), T, pairs),
                               f"graph replay splits={num_splits}")
            log(f"graph append+attend splits={num_splits}: 5 replays bit-identical, max abs err {err:.2e}")
    del g


def test_graph_fused_step_topk_and_noalloc():
    """kv_append_attend_q4 (the fused step), decode_attention_q4_topk without a workspace
    (one launch, scores on chip) and decode_attention_q4_noalloc with split partials in the
    library's static workspace, captured together in one graph."""
    require_gpu()
    b, a, d, s, n = 2, 4, 128, 700, 4
    cache, hc, q0 = _small_cache(b, a, d, s, n, 9400)
    cache2 = kvq.QuantKVCache(b, a, a * d, s, n, device=DEV, fill=0xFF)
    k = W.random_fp16((b, s + n, a, d), 9400, DEV)[:, :s].contiguous()   # the prompt rows of `cache`
    v = W.random_fp16((b, s + n, a, d), 9401, DEV)[:, :s].contiguous()
    kvq.kv_quantize_prefill(cache2, k, v)
    del k, v
    T = s + 1
    k_top = (T + 9) // 10
    kn = W.random_fp16((b, 1, a, d), 9403, DEV)
    vn = W.random_fp16((b, 1, a, d), 9404, DEV)
    kvq.kv_append_quant(cache, kn, vn, s)
    q = q0.clone()
    out_fused = torch.empty_like(q)
    out_topk = torch.empty_like(q)
    out_na = torch.empty_like(q)
    sel = torch.empty((b, a, k_top), dtype=torch.int32, device=DEV)
    assert kvq.kvq_workspace_bytes(cache, T, 0, k_top) == 0
    assert kvq.kvq_workspace_bytes(cache, T, 3, 0) > 0

    def step():
        kvq.kv_append_attend_q4(cache2, q, kn, vn, s, out=out_fused)
        kvq.decode_attention_q4_topk(cache, q, T, k_top, out=out_topk, sel_idx=sel)
        kvq.decode_attention_q4_noalloc(cache, q, T, out_na, num_splits=3)

    step()                                      # first use of every kernel and of the static workspace
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(5):
        q.copy_(W.random_fp16((b, 1, a, d), 9410 + i, DEV))
        for o in (out_fused, out_topk, out_na):
            o.fill_(float("nan"))
        sel.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_fused = kvq.decode_attention_q4(cache, q, T)
        ref_topk, ref_sel = kvq.decode_attention_q4_topk(cache, q, T, k_top)
        ref_split = kvq.decode_attention_q4(cache, q, T, num_splits=3)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_fused), _bits(ref_fused)), f"replay {i}: fused step"
        assert torch.equal(_bits(out_topk), _bits(ref_topk)) and torch.equal(sel, ref_sel), f"replay {i}: top-k"
        assert torch.equal(_bits(out_na), _bits(ref_split)), f"replay {i}: allocation-free call"
    log("graph fused step + top-k + noalloc: 5 replays bit-identical to the eager calls")
    del g
