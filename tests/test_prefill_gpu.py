"""GPU parity of the fused prefill (kv_quantize_prefill_attend) against the oracle.

Planes: bit-exact with the oracle's codec (binary32 and binary16 metadata) and
bit-identical to kv_quantize_prefill's; slots past the prompt untouched.
Attention: the oracle's binary64 causal prefill attention over the same fp16
Q, K, V, element-wise within 2e-3 + 1e-2 |oracle|.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_prefill_amd as kvq
import workloads as W
from tests.gpu_common import QUANTIZE, HostCache, _pool, assert_close, f16_np, log, require_gpu
from tests.test_parity_gpu import _check_prefill_full, _check_prefill_pairs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _oracle_rows(qh, kh, vh, pairs):
    """Oracle prefill attention of the given (bi, ai) pairs: [len(pairs)][s][d] (fp64)."""
    with _pool() as ex:
        return np.stack(list(ex.map(lambda p: oracle.prefill_attend(qh[p[0], :, p[1]], kh[p[0], :, p[1]],
                                                                    vh[p[0], :, p[1]]), pairs)))


def _gpu_pairs(out: torch.Tensor, pairs):
    o = out.float()
    return np.stack([o[bi, :, ai].cpu().numpy() for bi, ai in pairs])


def _run_small(b, a, d, s_len, S, seed, meta="f32", std=1.0):
    q = W.random_fp16((b, s_len, a, d), seed, DEV, std)
    k = W.random_fp16((b, s_len, a, d), seed + 1, DEV, std)
    v = W.random_fp16((b, s_len, a, d), seed + 2, DEV, std)
    cache = kvq.QuantKVCache(b, a, a * d, S, 0, device=DEV, fill=0xFF, meta=meta)
    out = torch.full_like(q, float("nan"))
    kvq.kv_quantize_prefill_attend(cache, q, k, v, out=out)
    torch.cuda.synchronize()
    return q, k, v, cache, out


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("s_len", [1, 17, 64, 65, 127, 128, 129, 300])
def test_prefill_small_full(d, s_len):
    """Every plane and every output: one and several query tiles, ragged last key and
    query tiles, the diagonal tiles, d = 64, 128, 256."""
    require_gpu()
    b, a = 2, 3
    q, k, v, cache, out = _run_small(b, a, d, s_len, s_len + 5, 7000 + d + s_len)
    hc = HostCache(b, a, d, s_len + 5)
    hc.prefill(f16_np(k), f16_np(v))
    _check_prefill_full(cache, hc, s_len, f"prefill d={d} s={s_len}")
    pairs = [(bi, ai) for bi in range(b) for ai in range(a)]
    ref = _oracle_rows(f16_np(q), f16_np(k), f16_np(v), pairs)
    err = assert_close(_gpu_pairs(out, pairs), ref, f"prefill attention d={d} s={s_len}")
    log(f"prefill d={d} s={s_len}: max abs err {err:.2e}")


@pytest.mark.parametrize("s_len", [17, 64, 200, 257])
def test_prefill_several_pairs_per_workgroup(s_len):
    """More (batch row, head) pairs (300) than workgroups at head_dim 128, so workgroups take
    a second pair: the tile ring and the early query fetch run across pair boundaries,
    including one-tile passes back to back (s <= 64) and a one-query last pass (s = 257).
    Every plane and every output row."""
    require_gpu()
    b, a, d = 3, 100, 128
    q, k, v, cache, out = _run_small(b, a, d, s_len, s_len + 3, 7600 + s_len)
    hc = HostCache(b, a, d, s_len + 3)
    hc.prefill(f16_np(k), f16_np(v))
    _check_prefill_full(cache, hc, s_len, f"prefill 300 pairs s={s_len}")
    pairs = [(bi, ai) for bi in range(b) for ai in range(a)]
    ref = _oracle_rows(f16_np(q), f16_np(k), f16_np(v), pairs)
    err = assert_close(_gpu_pairs(out, pairs), ref, f"prefill attention 300 pairs s={s_len}")
    log(f"prefill 300 pairs s={s_len}: max abs err {err:.2e}")


@pytest.mark.parametrize("d,s_len", [(64, 129), (128, 65), (256, 300)])
def test_prefill_small_full_m16(d, s_len):
    """Binary16 min/scale planes: every plane bit-exact with the oracle's binary16 codec and
    every output within the bar, at each head_dim."""
    require_gpu()
    b, a = 2, 3
    q, k, v, cache, out = _run_small(b, a, d, s_len, s_len + 3, 7500 + d + s_len, meta="f16")
    hc = HostCache(b, a, d, s_len + 3, "f16")
    hc.prefill(f16_np(k), f16_np(v))
    _check_prefill_full(cache, hc, s_len, f"prefill m16 d={d} s={s_len}")
    pairs = [(bi, ai) for bi in range(b) for ai in range(a)]
    ref = _oracle_rows(f16_np(q), f16_np(k), f16_np(v), pairs)
    assert_close(_gpu_pairs(out, pairs), ref, f"prefill m16 attention d={d} s={s_len}")


@pytest.mark.parametrize("meta", ["f32", "f16"])
def test_prefill_planes_equal_separate_quantiser_and_tail_untouched(meta):
    """The fused launch writes the same bytes as kv_quantize_prefill, and nothing past the
    prompt (slots s_len..S-1 keep their fill)."""
    require_gpu()
    b, a, d, s_len, S = 3, 4, 128, 333, 360
    q, k, v, c1, out = _run_small(b, a, d, s_len, S, 7100, meta=meta)
    c2 = kvq.QuantKVCache(b, a, a * d, S, 0, device=DEV, fill=0xFF, meta=meta)
    c0 = kvq.QuantKVCache(b, a, a * d, S, 0, device=DEV, fill=0xFF, meta=meta)  # never written
    kvq.kv_quantize_prefill(c2, k, v)
    torch.cuda.synchronize()
    for t1, t2, t0 in zip(c1.planes(), c2.planes(), c0.planes()):
        assert torch.equal(t1.view(torch.uint8), t2.view(torch.uint8))
        assert torch.equal(t1[:, :, s_len:].contiguous().view(torch.uint8),
                           t0[:, :, s_len:].contiguous().view(torch.uint8))
    hc = HostCache(b, a, d, S, meta)
    hc.prefill(f16_np(k), f16_np(v))
    _check_prefill_full(c1, hc, s_len, f"prefill planes meta={meta}")


@pytest.mark.parametrize("std", [4.0, 12.0])
def test_prefill_sharp_softmax(std):
    """Large q and k (scores of hundreds): near one-hot softmax rows, where the running
    max moves between key tiles."""
    require_gpu()
    b, a, d, s_len = 2, 2, 128, 200
    q, k, v, cache, out = _run_small(b, a, d, s_len, s_len, 7200 + int(std), std=std)
    pairs = [(bi, ai) for bi in range(b) for ai in range(a)]
    ref = _oracle_rows(f16_np(q), f16_np(k), f16_np(v), pairs)
    assert_close(_gpu_pairs(out, pairs), ref, f"prefill std={std}")


def test_prefill_deterministic():
    """Two launches give bit-identical outputs and planes."""
    require_gpu()
    b, a, d, s_len = 2, 3, 128, 257
    q, k, v, c1, o1 = _run_small(b, a, d, s_len, s_len, 7300)
    c2 = kvq.QuantKVCache(b, a, a * d, s_len, 0, device=DEV, fill=0, meta="f32")
    o2 = kvq.kv_quantize_prefill_attend(c2, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    for t1, t2 in zip(c1.planes(), c2.planes()):
        assert torch.equal(t1.view(torch.uint8), t2.view(torch.uint8))


@pytest.mark.timeout(600)
def test_prefill_batch_split_across_launches():
    """A prompt whose tensors exceed 2 GiB (b=48, a=96, d=128, s=2048: 2.4 GB each; eight
    256-query passes per pair): the kernel addresses each (batch row, head) from its own
    64-bit base with 32-bit offsets inside it.  Sampled pairs across the batch, including
    the first and last rows and heads and the rows around 2 GiB: planes bit-exact,
    attention within the bar."""
    require_gpu()
    b, a, d, s_len = 48, 96, 128, 2048
    log(f"[prefill split] b={b} a={a} d={d} s={s_len}")
    q = W.random_fp16((b, s_len, a, d), 7400, DEV)
    k = W.random_fp16((b, s_len, a, d), 7401, DEV)
    v = W.random_fp16((b, s_len, a, d), 7402, DEV)
    cache = kvq.QuantKVCache(b, a, a * d, s_len, 0, device=DEV, fill=0xFF)
    out = kvq.kv_quantize_prefill_attend(cache, q, k, v)
    torch.cuda.synchronize()
    pairs = [(0, 0), (41, 95), (42, 0), (42, 17), (47, 95), (20, 50)]
    hq = {p: q[p[0], :, p[1]].cpu().numpy() for p in pairs}
    hk = {p: k[p[0], :, p[1]].cpu().numpy() for p in pairs}
    hv = {p: v[p[0], :, p[1]].cpu().numpy() for p in pairs}
    hc = HostCache(b, a, d, s_len)
    for bi, ai in pairs:
        hc.kc[bi, ai], hc.kmin[bi, ai], hc.ksc[bi, ai] = QUANTIZE["f32"](hk[(bi, ai)].view(np.uint16))
        hc.vc[bi, ai], hc.vmin[bi, ai], hc.vsc[bi, ai] = QUANTIZE["f32"](hv[(bi, ai)].view(np.uint16))
    _check_prefill_pairs(cache, hc, s_len, pairs, "prefill split")
    with _pool() as ex:
        ref = np.stack(list(ex.map(lambda p: oracle.prefill_attend(hq[p], hk[p], hv[p]), pairs)))
    err = assert_close(_gpu_pairs(out, pairs), ref, "prefill split attention")
    log(f"[prefill split] {len(pairs)} pairs ok, max abs err {err:.2e}")


def _layer_sampled(w: W.Workload, meta: str, n_pairs: int, seed: int):
    require_gpu()
    log(f"[{w.name} prefill] b={w.b} a={w.a} d={w.d} s={w.s} meta={meta}")
    q = W.prefill_q(w, 0, DEV)
    k, v = W.prefill_kv(w, 0, DEV)
    cache = kvq.QuantKVCache(w.b, w.a, w.h, w.s, w.n, device=DEV, fill=0xFF, meta=meta)
    out = kvq.kv_quantize_prefill_attend(cache, q, k, v)
    torch.cuda.synchronize()
    r = np.random.default_rng(seed)
    idx = r.choice(w.b * w.a, size=n_pairs, replace=False)
    pairs = sorted({(0, 0), (w.b - 1, w.a - 1)} | {(int(i) // w.a, int(i) % w.a) for i in idx})
    hq = {p: q[p[0], :, p[1]].cpu().numpy() for p in pairs}
    hk = {p: k[p[0], :, p[1]].cpu().numpy() for p in pairs}
    hv = {p: v[p[0], :, p[1]].cpu().numpy() for p in pairs}
    hc = HostCache(w.b, w.a, w.d, w.S, meta)  # oracle planes of the sampled pairs only
    for bi, ai in pairs:
        c, m, s = QUANTIZE[meta](hk[(bi, ai)].view(np.uint16))
        hc.kc[bi, ai, :w.s], hc.kmin[bi, ai, :w.s], hc.ksc[bi, ai, :w.s] = c, m, s
        c, m, s = QUANTIZE[meta](hv[(bi, ai)].view(np.uint16))
        hc.vc[bi, ai, :w.s], hc.vmin[bi, ai, :w.s], hc.vsc[bi, ai, :w.s] = c, m, s
    _check_prefill_pairs(cache, hc, w.s, pairs, f"{w.name} prefill")
    with _pool() as ex:
        ref = np.stack(list(ex.map(lambda p: oracle.prefill_attend(hq[p], hk[p], hv[p]), pairs)))
    err = assert_close(_gpu_pairs(out, pairs), ref, f"{w.name} prefill attention")
    log(f"[{w.name} prefill] {len(pairs)} pairs: planes bit-exact, attention max abs err {err:.2e}")


@pytest.mark.timeout(600)
def test_prefill_opt175b_layer_sampled():
    """The OPT-175B layer (b=144, a=96, d=128, prompt 512) in the launch the benchmark
    times: 64 seeded (batch row, head) pairs plus the first and last, all 512 rows."""
    _layer_sampled(W.OPT_175B, "f32", 64, 91)


@pytest.mark.timeout(600)
def test_prefill_opt30b_layer_sampled_m16():
    """OPT-30B (b=256, a=56) with its outlier channels, binary16 planes: sampled pairs."""
    _layer_sampled(W.OPT_30B, "f16", 48, 92)


def _padded(shape, seed, slack_rows, std=1.0):
    """An fp16 tensor of `shape` at the front of a larger allocation whose remaining
    slack_rows token rows (a*d halves each) hold 0xFFFF, a binary16 NaN: any read past the
    tensor that reached the kernel's arithmetic would turn its outputs into NaN."""
    n = int(np.prod(shape))
    buf = torch.full((n + slack_rows * shape[2] * shape[3],), -1, dtype=torch.int16, device=DEV)
    x = buf[:n].view(torch.float16).view(shape)
    x.copy_(W.random_fp16(shape, seed, DEV, std))
    return x, buf


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("s_len", [100, 300])
def test_prefill_reads_nothing_past_the_prompt(d, s_len):
    """The last key tile of the last batch row reaches up to 63 token rows past the end of k
    and v.  With q, k and v at the front of allocations whose next 128 rows are NaN, every
    output stays finite and equals the oracle, and every plane is bit-exact: the rows past
    the prompt are read as zeros, not as the memory behind the tensors."""
    require_gpu()
    b, a = 3, 4
    shape = (b, s_len, a, d)
    seed = 7600 + d + s_len
    q, qb = _padded(shape, seed, 128)
    k, kb = _padded(shape, seed + 1, 128)
    v, vb = _padded(shape, seed + 2, 128)
    cache = kvq.QuantKVCache(b, a, a * d, s_len, 0, device=DEV, fill=0xFF)
    out = torch.full_like(q, float("nan"))
    kvq.kv_quantize_prefill_attend(cache, q, k, v, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    hc = HostCache(b, a, d, s_len)
    hc.prefill(f16_np(k), f16_np(v))
    _check_prefill_full(cache, hc, s_len, f"prefill padded d={d} s={s_len}")
    pairs = [(bi, ai) for bi in range(b) for ai in range(a)]
    ref = _oracle_rows(f16_np(q), f16_np(k), f16_np(v), pairs)
    assert_close(_gpu_pairs(out, pairs), ref, f"prefill padded d={d} s={s_len}")


@pytest.mark.parametrize("mode", ["all", "mixed"])
def test_prefill_subnormal_queries(mode):
    """Prompt queries holding binary16 subnormals (all of them, or about 10% mixed into
    N(0,1)): outputs against the oracle, which widens them exactly."""
    require_gpu()
    b, a, d, s_len = 2, 3, 128, 200
    r = np.random.default_rng(7700 + (mode == "all"))
    if mode == "all":
        qn = r.standard_normal((b, s_len, a, d)) * 1e-5
    else:
        qn = r.standard_normal((b, s_len, a, d))
        m = r.random(qn.shape) < 0.1
        qn[m] = r.standard_normal(int(m.sum())) * 2e-6
    q = torch.from_numpy(qn.astype(np.float16)).to(DEV)
    k = W.random_fp16((b, s_len, a, d), 7701, DEV)
    v = W.random_fp16((b, s_len, a, d), 7702, DEV)
    cache = kvq.QuantKVCache(b, a, a * d, s_len, 0, device=DEV, fill=0xFF)
    out = kvq.kv_quantize_prefill_attend(cache, q, k, v)
    torch.cuda.synchronize()
    pairs = [(bi, ai) for bi in range(b) for ai in range(a)]
    ref = _oracle_rows(f16_np(q), f16_np(k), f16_np(v), pairs)
    assert_close(_gpu_pairs(out, pairs), ref, f"prefill subnormal q ({mode})")


# query rows at the edges of the key tiles (64), the query tiles (128) and the prompt
PREFILL_ROWS = np.array([0, 1, 62, 63, 64, 65, 127, 128, 129, 191, 255, 256, 300, 383, 384, 447, 510, 511], np.int32)


@pytest.mark.timeout(900)
def test_prefill_opt175b_layer_all_pairs():
    """The OPT-175B layer (b=144, a=96, d=128, prompt 512) in the launch the benchmark times:
    all 13,824 (batch row, head) pairs at the query rows on every tile edge, against the
    oracle's causal attention at those rows; every prompt plane bit-exact."""
    require_gpu()
    w = W.OPT_175B
    log(f"[{w.name} prefill] b={w.b} a={w.a} d={w.d} s={w.s}: all pairs at {PREFILL_ROWS.size} rows")
    q = W.prefill_q(w, 0, DEV)
    k, v = W.prefill_kv(w, 0, DEV)
    cache = kvq.QuantKVCache(w.b, w.a, w.h, w.s, w.n, device=DEV, fill=0xFF)
    out = kvq.kv_quantize_prefill_attend(cache, q, k, v)
    torch.cuda.synchronize()
    qh, kh, vh = f16_np(q), f16_np(k), f16_np(v)
    del q, k, v
    hc = HostCache(w.b, w.a, w.d, w.S)
    hc.prefill(kh, vh)
    _check_prefill_full(cache, hc, w.s, f"{w.name} prefill")
    del hc
    rows_t = torch.from_numpy(PREFILL_ROWS.astype(np.int64)).to(DEV)
    got = out.index_select(1, rows_t).float().cpu().numpy()           # [b][rows][a][d]
    del out
    pairs = [(bi, ai) for bi in range(w.b) for ai in range(w.a)]

    def one(p):
        bi, ai = p
        return oracle.prefill_attend_rows(qh[bi, :, ai], kh[bi, :, ai], vh[bi, :, ai], PREFILL_ROWS)
    with _pool() as ex:
        ref = np.stack(list(ex.map(one, pairs)))                        # [pairs][rows][d]
    gpu = np.stack([got[bi, :, ai] for bi, ai in pairs])
    err = assert_close(gpu, ref, f"{w.name} prefill attention, all pairs")
    log(f"[{w.name} prefill] {len(pairs)} pairs x {PREFILL_ROWS.size} rows ok, planes bit-exact, "
        f"max abs err {err:.2e}")
