"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before anything is
enqueued (every call below fails validation, so no HIP launch happens).
"""
import ctypes
import os
import re

import pytest

import quantized_kv_cache_prefill_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq4.h")

KVQ_OK, KVQ_EINVAL, KVQ_ERANGE, KVQ_EUNSUPPORTED, KVQ_ENOSPACE, KVQ_ELAUNCH = 0, -1, -2, -3, -4, -5
FAKE = 0x10000  # aligned, non-null; never dereferenced because validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|void|size_t|char\s*\*|const char\s*\*)\s*\**\s*(\w+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    return kvq.load_library()


def test_header_declares_the_four_calls():
    fns = declared_functions()
    for f in ("kv_quantize_prefill", "kv_append_quant", "decode_attention_q4", "decode_attention_q4_topk"):
        assert f in fns
    assert set(kvq.EXPORTED) == set(fns)


def test_library_exports_every_declared_symbol(L):
    for f in declared_functions():
        assert hasattr(L, f), f


def test_library_links_no_oracle():
    data = open(kvq.library_path(), "rb").read()
    assert b"oracle_" not in data


def dims(b=2, a=2, h=128, s=16, n=4, group=64, meta=0):
    return kvq.KvqDims(b, a, h, s, n, group, meta)


def cache(d=None, ptrs=(FAKE,) * 6):
    d = dims() if d is None else d
    return kvq.KvqCache(d, *ptrs)


def test_cache_bytes_closed_form(L):
    """One layer: codes = 2 planes x 0.5 byte x h x (s+n) x b (the blog's KV-cache size with
    precision 0.5 and one layer); metadata = (h/64) groups x 4 bytes, per plane."""
    for (b, a, h, s, n) in [(2, 2, 128, 16, 4), (144, 96, 12288, 512, 32), (256, 56, 7168, 512, 32)]:
        cb, mb = kvq.kvq_cache_bytes(b, a, h, s, n)
        assert 2 * cb == 2 * 0.5 * h * (s + n) * b
        assert mb == b * (s + n) * (h // 64) * 4
        cb16, mb16 = kvq.kvq_cache_bytes(b, a, h, s, n, meta="f16")
        assert cb16 == cb and mb16 == b * (s + n) * (h // 64) * 2
    # OPT-175B layer at d = 128: 160 bytes per (batch row, head, token) with binary32 planes, 144 with binary16
    cb, mb = kvq.kvq_cache_bytes(144, 96, 12288, 512, 32)
    cb16, mb16 = kvq.kvq_cache_bytes(144, 96, 12288, 512, 32, meta="f16")
    slots = 144 * 96 * 544
    assert (2 * cb + 4 * mb) == 160 * slots and (2 * cb16 + 4 * mb16) == 144 * slots


@pytest.mark.parametrize("mut,status", [
    (dict(b=0), KVQ_EINVAL), (dict(a=0), KVQ_EINVAL), (dict(h=100), KVQ_EINVAL), (dict(s=0), KVQ_EINVAL),
    (dict(h=2 * 96), KVQ_EINVAL), (dict(group=32), KVQ_EUNSUPPORTED), (dict(meta=2), KVQ_EUNSUPPORTED),
    (dict(meta=-1), KVQ_EUNSUPPORTED),
    (dict(h=2 * 192), KVQ_EUNSUPPORTED), (dict(h=2 * 512), KVQ_EUNSUPPORTED), (dict(n=-1), KVQ_EINVAL),
])
def test_bad_dims(L, mut, status):
    d = dims(**mut)
    cb = ctypes.c_size_t()
    assert L.kvq_cache_bytes(ctypes.byref(d), ctypes.byref(cb), None) == status
    c = cache(d)
    st = ctypes.c_void_p(0)
    assert L.kv_quantize_prefill(ctypes.byref(c), FAKE, FAKE, 4, st) == status
    assert L.kv_append_quant(ctypes.byref(c), FAKE, FAKE, 0, st) == status
    assert L.decode_attention_q4(ctypes.byref(c), FAKE, 4, FAKE, 0, None, 0, st) == status
    assert L.decode_attention_q4_topk(ctypes.byref(c), FAKE, 4, 1, FAKE, None, None, 0, st) == status
    assert L.kvq_workspace_bytes(ctypes.byref(d), 4, 0, 0) == 0


@pytest.mark.parametrize("h,a,S,ok", [
    (256, 1, (1 << 24) - 1, True), (256, 1, 1 << 24, False),       # d = 256: S * 128 < 2^31
    (128, 1, (1 << 25) - 1, True), (128, 1, 1 << 25, False),       # d = 128: S * 64 < 2^31
    (64, 1, (1 << 26) - 1, True), (64, 1, 1 << 26, False),         # d = 64: S * 32 < 2^31
    (12288, 96, 1 << 25, False), (12288, 96, 544, True),
])
def test_slot_offsets_fit_31_bits(L, h, a, S, ok):
    """The attention kernels address one (batch row, head)'s code rows with 32-bit byte
    offsets: a cache with S * d/2 >= 2^31 is refused by every call (KVQ_EUNSUPPORTED), before
    anything is enqueued, for every call that takes a cache and for the sizing calls."""
    d = dims(b=1, a=a, h=h, s=S - 1, n=1)
    cb = ctypes.c_size_t()
    want = KVQ_OK if ok else KVQ_EUNSUPPORTED
    assert L.kvq_cache_bytes(ctypes.byref(d), ctypes.byref(cb), None) == want
    if ok:
        assert cb.value == S * (h // a) // 2 * a
        return
    c = cache(d)
    st = ctypes.c_void_p(0)
    assert L.kvq_workspace_bytes(ctypes.byref(d), 4, 0, 0) == 0
    assert L.kv_quantize_prefill(ctypes.byref(c), FAKE, FAKE, 4, st) == KVQ_EUNSUPPORTED
    assert L.kv_quantize_prefill_attend(ctypes.byref(c), FAKE, FAKE, FAKE, 4, FAKE, st) == KVQ_EUNSUPPORTED
    assert L.kv_append_quant(ctypes.byref(c), FAKE, FAKE, S - 1, st) == KVQ_EUNSUPPORTED
    assert L.decode_attention_q4(ctypes.byref(c), FAKE, S, FAKE, 0, FAKE, 1 << 30, st) == KVQ_EUNSUPPORTED
    assert L.decode_attention_q4_tuned(ctypes.byref(c), FAKE, S, FAKE, 0, 4, 2, FAKE, 1 << 30, st) == KVQ_EUNSUPPORTED
    assert L.kv_append_attend_q4(ctypes.byref(c), FAKE, FAKE, FAKE, S - 1, FAKE, 0, FAKE, 1 << 30,
                                 st) == KVQ_EUNSUPPORTED
    assert L.decode_attention_q4_topk(ctypes.byref(c), FAKE, 4, 1, FAKE, None, FAKE, 1 << 30,
                                      st) == KVQ_EUNSUPPORTED
    assert L.kv_quantize_prefill_host(ctypes.byref(c), FAKE, FAKE, 4, 1) == KVQ_EUNSUPPORTED
    assert L.decode_attention_q4_host(ctypes.byref(c), FAKE, 4, FAKE, 1) == KVQ_EUNSUPPORTED


def test_null_and_misaligned_pointers(L):
    st = ctypes.c_void_p(0)
    assert L.kv_quantize_prefill(None, FAKE, FAKE, 4, st) == KVQ_EINVAL
    for i in range(6):
        ptrs = [FAKE] * 6
        ptrs[i] = 0
        assert L.kv_quantize_prefill(ctypes.byref(cache(ptrs=ptrs)), FAKE, FAKE, 4, st) == KVQ_EINVAL
        ptrs[i] = FAKE + 4
        assert L.decode_attention_q4(ctypes.byref(cache(ptrs=ptrs)), FAKE, 4, FAKE, 0, None, 0, st) == KVQ_EINVAL
    c = cache()
    assert L.kv_quantize_prefill(ctypes.byref(c), None, FAKE, 4, st) == KVQ_EINVAL
    assert L.kv_quantize_prefill(ctypes.byref(c), FAKE, FAKE + 2, 4, st) == KVQ_EINVAL
    assert L.kv_append_quant(ctypes.byref(c), FAKE, None, 0, st) == KVQ_EINVAL
    assert L.decode_attention_q4(ctypes.byref(c), None, 4, FAKE, 0, None, 0, st) == KVQ_EINVAL
    assert L.decode_attention_q4(ctypes.byref(c), FAKE, 4, FAKE + 8, 0, None, 0, st) == KVQ_EINVAL
    assert L.decode_attention_q4_topk(ctypes.byref(c), FAKE, 4, 1, None, None, FAKE, 1 << 20, st) == KVQ_EINVAL
    assert L.decode_attention_q4_topk(ctypes.byref(c), FAKE, 4, 1, FAKE, FAKE + 2, FAKE, 1 << 20, st) == KVQ_EINVAL
    assert L.decode_attention_q4_topk(ctypes.byref(c), FAKE, 4, 1, FAKE, None, FAKE + 4, 1 << 20, st) == KVQ_EINVAL


def test_ranges(L):
    st = ctypes.c_void_p(0)
    c = cache()  # S = 20
    assert L.kv_quantize_prefill(ctypes.byref(c), FAKE, FAKE, 0, st) == KVQ_ERANGE
    assert L.kv_quantize_prefill(ctypes.byref(c), FAKE, FAKE, 21, st) == KVQ_ERANGE
    assert L.kv_append_quant(ctypes.byref(c), FAKE, FAKE, -1, st) == KVQ_ERANGE
    assert L.kv_append_quant(ctypes.byref(c), FAKE, FAKE, 20, st) == KVQ_ERANGE
    assert L.decode_attention_q4(ctypes.byref(c), FAKE, 0, FAKE, 0, None, 0, st) == KVQ_ERANGE
    assert L.decode_attention_q4(ctypes.byref(c), FAKE, 21, FAKE, 0, None, 0, st) == KVQ_ERANGE
    assert L.decode_attention_q4(ctypes.byref(c), FAKE, 4, FAKE, -1, None, 0, st) == KVQ_ERANGE
    assert L.decode_attention_q4(ctypes.byref(c), FAKE, 4, FAKE, 257, None, 0, st) == KVQ_ERANGE
    assert L.decode_attention_q4_tuned(ctypes.byref(c), FAKE, 4, FAKE, 1, 3, 1, None, 0, st) == KVQ_EINVAL
    assert L.decode_attention_q4_tuned(ctypes.byref(c), FAKE, 4, FAKE, 1, 2, 8, None, 0, st) == KVQ_EINVAL
    assert L.decode_attention_q4_tuned(ctypes.byref(c), FAKE, 4, FAKE, 1, 4, 0, None, 0, st) == KVQ_EINVAL
    assert L.decode_attention_q4_topk(ctypes.byref(c), FAKE, 10, 0, FAKE, None, None, 0, st) == KVQ_ERANGE
    assert L.decode_attention_q4_topk(ctypes.byref(c), FAKE, 10, 11, FAKE, None, None, 0, st) == KVQ_ERANGE
    big = cache(dims(s=9000, n=0))
    assert L.decode_attention_q4_topk(ctypes.byref(big), FAKE, 8193, 5, FAKE, None, None, 0, st) == KVQ_EUNSUPPORTED


def test_workspace_sizing_and_enospace(L):
    st = ctypes.c_void_p(0)
    d = dims(b=1, a=1, h=128, s=4000, n=96)
    c = cache(d)
    # one split: no workspace
    assert L.kvq_workspace_bytes(ctypes.byref(d), 100, 1, 0) == 0
    # explicit splits: splits x pairs x (d + 2) floats
    assert L.kvq_workspace_bytes(ctypes.byref(d), 4096, 7, 0) == 7 * 1 * 130 * 4
    # automatic: a single (batch row, head) with a long context is split
    auto = L.kvq_workspace_bytes(ctypes.byref(d), 4096, 0, 0)
    assert auto > 0 and auto % (130 * 4) == 0
    assert L.decode_attention_q4(ctypes.byref(c), FAKE, 4096, FAKE, 7, FAKE, 7 * 130 * 4 - 4, st) == KVQ_ENOSPACE
    assert L.decode_attention_q4(ctypes.byref(c), FAKE, 4096, FAKE, 7, None, 0, st) == KVQ_ENOSPACE
    # the top-k path: up to KVQ_TOPK_FUSED_MAX_CTX tokens one launch keeps the scores on chip
    # (no workspace needed; one that is given must hold them); beyond, it holds one fp32 score
    # per (pair, token) between its two kernels
    assert kvq.KVQ_TOPK_FUSED_MAX_CTX == 2048
    assert L.kvq_workspace_bytes(ctypes.byref(d), 2048, 0, 205) == 0
    assert L.kvq_workspace_bytes(ctypes.byref(d), 2049, 0, 205) == 1 * 1 * 2049 * 4
    assert L.decode_attention_q4_topk(ctypes.byref(c), FAKE, 2048, 205, FAKE, None, FAKE, 2048 * 4 - 4,
                                      st) == KVQ_ENOSPACE
    assert L.decode_attention_q4_topk(ctypes.byref(c), FAKE, 2048, 205, FAKE, None, FAKE + 4, 2048 * 4,
                                      st) == KVQ_EINVAL
    assert L.decode_attention_q4_topk(ctypes.byref(c), FAKE, 2049, 205, FAKE, None, FAKE, 2049 * 4 - 4,
                                      st) == KVQ_ENOSPACE
    assert L.decode_attention_q4_topk(ctypes.byref(c), FAKE, 2049, 205, FAKE, None, None, 0, st) == KVQ_ENOSPACE


def test_append_attend_validation(L):
    st = ctypes.c_void_p(0)
    c = cache()  # S = 20
    assert L.kv_append_attend_q4(None, FAKE, FAKE, FAKE, 0, FAKE, 0, None, 0, st) == KVQ_EINVAL
    assert L.kv_append_attend_q4(ctypes.byref(c), FAKE, None, FAKE, 0, FAKE, 0, None, 0, st) == KVQ_EINVAL
    assert L.kv_append_attend_q4(ctypes.byref(c), FAKE, FAKE, FAKE + 2, 0, FAKE, 0, None, 0, st) == KVQ_EINVAL
    assert L.kv_append_attend_q4(ctypes.byref(c), FAKE, FAKE, FAKE, -1, FAKE, 0, None, 0, st) == KVQ_ERANGE
    assert L.kv_append_attend_q4(ctypes.byref(c), FAKE, FAKE, FAKE, 20, FAKE, 0, None, 0, st) == KVQ_ERANGE
    assert L.kv_append_attend_q4(ctypes.byref(cache(dims(group=32))), FAKE, FAKE, FAKE, 0, FAKE, 0, None, 0,
                                 st) == KVQ_EUNSUPPORTED
    d = dims(b=1, a=1, h=128, s=4000, n=96)
    assert L.kv_append_attend_q4(ctypes.byref(cache(d)), FAKE, FAKE, FAKE, 4095, FAKE, 7, None, 0, st) == KVQ_ENOSPACE


def test_prefill_attend_validation(L):
    """kv_quantize_prefill_attend: bad dims, NULL or misaligned q/k/v/out, s_len outside
    1..S are rejected on the host before any launch."""
    st = ctypes.c_void_p(0)
    c = cache()  # S = 20
    f = L.kv_quantize_prefill_attend
    assert f(None, FAKE, FAKE, FAKE, 4, FAKE, st) == KVQ_EINVAL
    for i in range(4):
        ptrs = [FAKE] * 4
        ptrs[i] = 0
        assert f(ctypes.byref(c), *ptrs[:3], 4, ptrs[3], st) == KVQ_EINVAL
        ptrs[i] = FAKE + 2
        assert f(ctypes.byref(c), *ptrs[:3], 4, ptrs[3], st) == KVQ_EINVAL
    assert f(ctypes.byref(c), FAKE, FAKE, FAKE, 0, FAKE, st) == KVQ_ERANGE
    assert f(ctypes.byref(c), FAKE, FAKE, FAKE, 21, FAKE, st) == KVQ_ERANGE
    bad = cache(dims(h=96 * 3))  # head_dim 3 is not a multiple of 64
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, 4, FAKE, st) != KVQ_OK
    # one batch row of a 90,000-token prompt at h = 12288 exceeds 31-bit byte offsets
    long = cache(dims(b=1, a=96, h=12288, s=90000, n=0))
    assert f(ctypes.byref(long), FAKE, FAKE, FAKE, 90000, FAKE, st) == KVQ_EUNSUPPORTED


def test_auto_splits_only_when_the_pairs_cannot_fill_the_card(L):
    """Automatic split choice (read through the workspace size, 0 when one split): many
    pairs -> one split whatever the round count; few pairs over a long context -> splits."""
    for b in (128, 136, 144, 171, 256):
        d = dims(b=b, a=96, h=12288, s=512, n=32)
        assert L.kvq_workspace_bytes(ctypes.byref(d), 544, 0, 0) == 0, b
    long = dims(b=1, a=96, h=12288, s=65536, n=0)
    assert L.kvq_workspace_bytes(ctypes.byref(long), 65536, 0, 0) > 0


@pytest.mark.parametrize("b,a,ctx,splits", [
    (16, 32, 544, 1),      # 512 pairs: four waves each, 2,048 waves, no split
    (4, 32, 544, 1),       # 128 pairs: splits would be shorter than 512 tokens
    (4, 32, 2048, 2),      # 128 pairs: two splits make 1,024 waves
    (1, 32, 4096, 8),      # 32 pairs: eight splits of 512 tokens
    (1, 32, 16384, 8),     # 32 pairs: 1,024 waves
    (1, 96, 65536, 8),     # 96 pairs: no wave streams more than 2,048 tokens
    (1, 1, 4096, 8),       # one pair: as many 512-token splits as the context holds
    (31, 33, 544, 1),      # 1,023 pairs, the last of the few-pairs range
])
def test_auto_shape_for_few_pairs(L, b, a, ctx, splits):
    """Fewer pairs than fill every CU with two workgroups of two-wave pairs: four waves per
    pair and splits until the launch has 1,024 waves or no wave streams more than 2,048
    tokens, each split at least 512 tokens.  Read through the workspace size: splits x
    pairs x (d + 2) floats, 0 for one split."""
    d = dims(b=b, a=a, h=a * 128, s=ctx, n=0)
    want = 0 if splits == 1 else splits * b * a * 130 * 4
    assert L.kvq_workspace_bytes(ctypes.byref(d), ctx, 0, 0) == want


def test_strerror(L):
    for s in (0, -1, -2, -3, -4, -5, -99):
        assert len(L.kvq_strerror(s)) > 0


def test_gemm_w4_validation_and_workspace(L):
    st = ctypes.c_void_p(0)
    # shapes: N % 64, K % 128, M >= 1
    for (M, N, K) in [(0, 64, 128), (1, 63, 128), (1, 64, 64), (1, 100, 128), (4, 64, 192)]:
        assert L.gemm_w4a16(FAKE, M, N, K, FAKE, FAKE, FAKE, FAKE, 0, None, 0, st) == KVQ_EINVAL
        assert L.kvq_gemm_w4_workspace_bytes(M, N, K, 0) == 0
    assert L.kvq_w4_quantize(FAKE, 64, 96, FAKE, FAKE, FAKE, st) == KVQ_EINVAL
    assert L.kvq_w4_quantize(None, 64, 128, FAKE, FAKE, FAKE, st) == KVQ_EINVAL
    assert L.kvq_w4_quantize(FAKE, 64, 128, FAKE, FAKE + 2, FAKE, st) == KVQ_EINVAL
    assert L.gemm_w4a16(None, 1, 64, 128, FAKE, FAKE, FAKE, FAKE, 0, None, 0, st) == KVQ_EINVAL
    assert L.gemm_w4a16(FAKE, 1, 64, 128, FAKE, FAKE, FAKE, FAKE + 8, 0, None, 0, st) == KVQ_EINVAL
    # num_splits range: KVQ_GEMM_STREAM (-1), 0 (auto) .. K/128
    assert L.gemm_w4a16(FAKE, 1, 64, 256, FAKE, FAKE, FAKE, FAKE, 3, FAKE, 1 << 20, st) == KVQ_ERANGE
    assert L.gemm_w4a16(FAKE, 1, 64, 256, FAKE, FAKE, FAKE, FAKE, -2, FAKE, 1 << 20, st) == KVQ_ERANGE
    assert L.kvq_gemm_w4_workspace_bytes(1, 64, 256, -2) == 0
    # stream form: min(256, units / 4) workgroups (units = tiles x K/128), two binary32 partial tiles of
    # (32 x row blocks) x 256 each
    assert L.kvq_gemm_w4_workspace_bytes(144, 36864, 12288, -1) == 256 * 2 * 160 * 256 * 4
    assert L.kvq_gemm_w4_workspace_bytes(33, 1280, 384, -1) == 3 * 2 * 64 * 256 * 4
    assert L.kvq_gemm_w4_workspace_bytes(1, 64, 256, -1) == 1 * 2 * 32 * 256 * 4
    assert L.gemm_w4a16(FAKE, 33, 1280, 384, FAKE, FAKE, FAKE, FAKE, -1, FAKE, 3 * 2 * 64 * 256 * 4 - 4,
                        st) == KVQ_ENOSPACE
    # explicit splits: splits x M x N binary32 partials
    assert L.kvq_gemm_w4_workspace_bytes(144, 256, 1024, 1) == 0
    assert L.kvq_gemm_w4_workspace_bytes(144, 256, 1024, 4) == 4 * 144 * 256 * 4
    assert L.gemm_w4a16(FAKE, 144, 256, 1024, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 4 * 144 * 256 * 4 - 4,
                        st) == KVQ_ENOSPACE
    assert L.gemm_w4a16(FAKE, 144, 256, 1024, FAKE, FAKE, FAKE, FAKE, 4, None, 0, st) == KVQ_ENOSPACE
    # automatic: the OPT-175B decode projection (M=144, N=K=12288) splits K over the 48 column tiles
    auto = L.kvq_gemm_w4_workspace_bytes(144, 12288, 12288, 0)
    assert auto > 0 and auto % (144 * 12288 * 4) == 0
    # automatic choices on the OPT-175B projections (K = 12288, 96 chunks of 128): the output projection
    # (48 column tiles) takes 5 splits at every M -- 240 workgroups, one round; QKV (N = 36864, 144
    # column tiles) would need more than one round of workgroups at any split count >= 2 and takes the
    # stream form (256 workgroups, two partial tiles of 32 x row blocks each); so do M = 150 (one row
    # tile of 160 rows) and M = 161 (two row tiles, 288 tiles: two rounds even unsplit)
    for M, N, splits in [(144, 12288, 5), (64, 12288, 5), (32, 12288, 5), (1, 12288, 5)]:
        assert L.kvq_gemm_w4_workspace_bytes(M, N, 12288, 0) == splits * M * N * 4, (M, N)
    for M, rows in [(144, 160), (64, 64), (32, 32), (16, 32), (1, 32), (150, 160), (161, 160)]:
        want = 256 * 2 * rows * 256 * 4
        assert L.kvq_gemm_w4_workspace_bytes(M, 36864, 12288, 0) == want, M
        assert L.kvq_gemm_w4_workspace_bytes(M, 36864, 12288, -1) == want, M
    # 32-column x 64-row weight (N = 64, K = 128): one unit, one workgroup, one round: unsplit
    assert L.kvq_gemm_w4_workspace_bytes(1, 64, 128, 0) == 0
    # the stream form's 32-bit unit range: units x workgroups < 2^32, else refused (workspace 0)
    big_m = 160 * 100000  # 100000 row tiles x 256 column tiles x 1 chunk = 25.6M units; x 256 >= 2^32
    assert L.kvq_gemm_w4_workspace_bytes(big_m, 65536, 128, -1) == 0
    assert L.gemm_w4a16(FAKE, big_m, 65536, 128, FAKE, FAKE, FAKE, FAKE, -1, FAKE, 1 << 40, st) == KVQ_ERANGE
    assert L.kvq_gemm_w4_workspace_bytes(big_m, 65536, 128, 0) == 0  # automatic: unsplit
    # a split count that leaves an empty split is reduced: 96 chunks in 7 splits -> 14 per split, 7 splits
    assert L.kvq_gemm_w4_workspace_bytes(1, 64, 12288, 7) == 7 * 64 * 4
    assert L.kvq_gemm_w4_workspace_bytes(1, 64, 12288, 95) == 48 * 64 * 4  # ceil(96/95)=2 chunks each -> 48 splits


def test_noalloc_refusals_before_any_launch(L):
    """decode_attention_q4_noalloc checks everything on the host first: bad dimensions and
    ranges as decode_attention_q4 does, and a launch whose split partials exceed the static
    workspace (KVQ_NOALLOC_SCRATCH_BYTES) is KVQ_ENOSPACE -- no device is touched."""
    st = ctypes.c_void_p(0)
    big = cache(dims(b=64, a=32, h=32 * 256, s=8192, n=0))
    d = big.dims
    assert L.kvq_workspace_bytes(ctypes.byref(d), 8192, 256, 0) > kvq.KVQ_NOALLOC_SCRATCH_BYTES
    assert L.decode_attention_q4_noalloc(ctypes.byref(big), FAKE, 8192, FAKE, 256, st) == KVQ_ENOSPACE
    c = cache()
    assert L.decode_attention_q4_noalloc(ctypes.byref(c), FAKE, 0, FAKE, 0, st) == KVQ_ERANGE
    assert L.decode_attention_q4_noalloc(ctypes.byref(c), FAKE, 21, FAKE, 0, st) == KVQ_ERANGE
    assert L.decode_attention_q4_noalloc(ctypes.byref(c), FAKE, 4, FAKE, 257, st) == KVQ_ERANGE
    assert L.decode_attention_q4_noalloc(ctypes.byref(c), None, 4, FAKE, 0, st) == KVQ_EINVAL
    assert L.decode_attention_q4_noalloc(ctypes.byref(c), FAKE, 4, FAKE + 2, 0, st) == KVQ_EINVAL
    assert L.decode_attention_q4_noalloc(None, FAKE, 4, FAKE, 0, st) == KVQ_EINVAL


def test_codec_params_refusals_before_any_launch(L):
    """kvq_codec_params checks its arguments on the host: NULL or misaligned pointers are
    KVQ_EINVAL, an unknown metadata type KVQ_EUNSUPPORTED, a negative count KVQ_ERANGE; a
    count of 0 enqueues nothing."""
    st = ctypes.c_void_p(0)
    assert L.kvq_codec_params(None, 16, 0, FAKE, FAKE, st) == KVQ_EINVAL
    assert L.kvq_codec_params(FAKE, 16, 0, FAKE + 2, FAKE, st) == KVQ_EINVAL
    assert L.kvq_codec_params(FAKE, 16, 0, FAKE, None, st) == KVQ_EINVAL
    assert L.kvq_codec_params(FAKE, 16, 7, FAKE, FAKE, st) == KVQ_EUNSUPPORTED
    assert L.kvq_codec_params(FAKE, -1, 0, FAKE, FAKE, st) == KVQ_ERANGE
    assert L.kvq_codec_params(FAKE, 0, 1, None, None, st) == KVQ_OK
