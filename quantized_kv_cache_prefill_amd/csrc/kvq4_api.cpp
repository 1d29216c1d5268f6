// C-ABI layer: argument checks (all on the host, before anything is
// enqueued), launch-shape choice, and the calls into the HIP kernels.
// The operations and their sources on the pages are documented in
// include/kvq4.h.
#include "kvq4.h"

#include <stdint.h>

#include <algorithm>
#include <cmath>

#include <hip/hip_runtime_api.h>

#include "kvq4_launch.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by every call; fills the kernel-side view of the cache.
int check_dims(const kvq_dims *d)
{
    if (d == nullptr)
        return KVQ_EINVAL;
    if (d->b <= 0 || d->a <= 0 || d->h <= 0 || d->s <= 0 || d->n < 0)
        return KVQ_EINVAL;
    if (d->h % d->a != 0)
        return KVQ_EINVAL;
    const int hd = d->h / d->a;
    if (hd % KVQ_GROUP != 0)
        return KVQ_EINVAL;
    if (d->group != KVQ_GROUP || (d->meta_dtype != KVQ_META_F32 && d->meta_dtype != KVQ_META_F16))
        return KVQ_EUNSUPPORTED;
    if (hd != 64 && hd != 128 && hd != 256)
        return KVQ_EUNSUPPORTED;
    if ((int64_t)d->s + d->n > INT32_MAX / 2)
        return KVQ_ERANGE;
    if ((int64_t)d->b * d->a > INT32_MAX / 4)
        return KVQ_ERANGE;
    // The attention kernels address the tokens of one (batch row, head) with
    // 32-bit byte offsets into its code rows: S * d/2 must stay below 2^31.
    if (((int64_t)d->s + d->n) * (hd / 2) >= ((int64_t)1 << 31))
        return KVQ_EUNSUPPORTED;
    return KVQ_OK;
}

int check_cache(const kvq_cache *c, kvq::CachePlanes *planes)
{
    if (c == nullptr)
        return KVQ_EINVAL;
    int st = check_dims(&c->dims);
    if (st != KVQ_OK)
        return st;
    const void *ptrs[6] = {c->k_codes, c->v_codes, c->k_min, c->k_scale, c->v_min, c->v_scale};
    for (const void *p : ptrs)
        if (p == nullptr || !aligned16(p))
            return KVQ_EINVAL;
    planes->k_codes = c->k_codes;
    planes->v_codes = c->v_codes;
    planes->k_min = c->k_min;
    planes->k_scale = c->k_scale;
    planes->v_min = c->v_min;
    planes->v_scale = c->v_scale;
    planes->a = c->dims.a;
    planes->d = c->dims.h / c->dims.a;
    planes->S = c->dims.s + c->dims.n;
    planes->meta_f16 = c->dims.meta_dtype == KVQ_META_F16;
    return KVQ_OK;
}

int check_act(const void *p) { return (p == nullptr || !aligned16(p)) ? KVQ_EINVAL : KVQ_OK; }

int status_of(int hip_err) { return hip_err == 0 ? KVQ_OK : KVQ_ELAUNCH; }

// Launch shape for the dense decode kernel.  Default: 4 token rows per lane
// per iteration and 2 waves per (batch row, head), two pairs per 256-thread
// workgroup -- the fastest shape of the measured sweeps on the OPT-175B layer
// (191.8 us against 197.1 us for 4 waves per pair at context 544).
constexpr int kDefaultUnroll = 4;
constexpr int kDefaultWavesPerPair = 2;
constexpr int kPairsPerGroup = 4 / kDefaultWavesPerPair;
// Automatic launch shape: an unsplit context of at least this many tokens is
// shared by four waves per (batch row, head) instead of two (measured on
// MI355X: b=32 a=96 T=2048 170.7 -> 159.7 us, b=64 a=32 T=2048 118.1 ->
// 108.9 us, b=144 a=96 T=1024 level within 1.4%; with splits, or below 1536
// tokens, two waves were level or faster).
constexpr int kLongCtxFourWaves = 1536;
constexpr int kAutoWavesPerPair = 0;

// Automatic split count.  The split workgroups of all pairs should spread
// evenly over MI355X's 256 CUs with at least two workgroups (8 waves) per CU:
// with x = workgroups / 256, efficiency e = (x / ceil(x)) * min(1, x / 2),
// and the smallest split count with the best e wins (measured: 11 splits of
// 48 workgroup groups = 2.06 per CU ran 30% slower than 16 splits = 3 per
// CU).  A split covers a whole number of 128-token blocks, so every wave
// starts on a 128-byte boundary of the code and min/scale planes, and is at
// least 256 tokens long.  The choice depends on (pairs, ctx) only, so
// kvq_workspace_bytes() is exact for every launch shape.
constexpr int kCUs = 256;
constexpr int kSplitAlign = 128;
constexpr int kMaxAutoSplits = 64;

// Fewer pairs than give every CU two workgroups of two-wave pairs: four waves
// per pair, and splits until the launch has 1,024 waves (4 per CU) and no
// wave streams more than 512 tokens, but no more than 3,072 waves (12 per
// CU) and no split shorter than 512 tokens.  Measured on MI355X, HBM-cold,
// 32..768 pairs at contexts 544..65536, against 1..32 splits with two or
// four waves per pair: short contexts gain most from few splits (the reduce
// pass and the partials are then a large part of the call), long ones from
// about 512 tokens per wave (32 pairs at 16384 tokens: 8 splits, 27.0 us
// against 38.1 us for the balance rule below; 512 pairs at 544 tokens: no
// split, 14.9 against 18.8 us).
constexpr int kFewPairs = 2 * kCUs * kPairsPerGroup;
constexpr int kFewPairsMinWaves = 4 * kCUs;
constexpr int kFewPairsMaxWaves = 12 * kCUs;
constexpr int kFewPairsWaveTokens = 512;
constexpr int kFewPairsMinSplit = 512;

int resolve_splits(int pairs, int ctx, int num_splits, int *split_len)
{
    int s;
    if (num_splits > 0) {
        s = num_splits;
    } else if (pairs < kFewPairs) {
        const int by_waves = (kFewPairsMinWaves + 4 * pairs - 1) / (4 * pairs);
        const int by_length = (ctx + 4 * kFewPairsWaveTokens - 1) / (4 * kFewPairsWaveTokens);
        s = std::min(std::max(by_waves, by_length), std::max(1, kFewPairsMaxWaves / (4 * pairs)));
        s = std::min(s, std::max(1, std::min(ctx / kFewPairsMinSplit, kMaxAutoSplits)));
    } else {
        const int64_t groups = (pairs + kPairsPerGroup - 1) / kPairsPerGroup;
        // With at least four workgroups per CU there is parallelism enough and the
        // last round is a small part of the launch: a split would only add the
        // partials' traffic and the reduce pass (measured on MI355X: 2 splits at
        // 6,528 workgroups ran 25% slower than one).
        const int cap = groups >= 4 * kCUs
                            ? 1
                            : (int)std::max<int64_t>(1, std::min<int64_t>(ctx / (2 * kSplitAlign), kMaxAutoSplits));
        s = 1;
        double best = -1.0;
        for (int c = 1; c <= cap; ++c) {
            const double x = (double)(groups * c) / kCUs;
            const double e = x / std::ceil(x) * std::min(1.0, x / 2.0);
            if (e > best + 1e-9) {
                best = e;
                s = c;
            }
        }
    }
    s = std::min(s, ctx);
    int len = (ctx + s - 1) / s;
    if (s > 1)
        len = (len + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
    s = (ctx + len - 1) / len; // no empty split
    *split_len = len;
    return s;
}

// Split of the K range for gemm_w4a16: as many splits as give every CU one
// workgroup (a second workgroup on a CU shares its matrix core and vector
// ALU, so it adds no throughput), with at least 4 chunks of 128 k per split;
// when that leaves one split of an under-filled round, the split count that
// minimises (rounds x each split's share of K) + a cost for the partials.
// Depends on (M, N, K) only.
constexpr int kGemmChunk = 128;
constexpr int kGemmCols = 256;

bool gemm_dims_ok(int M, int N, int K)
{
    return M >= 1 && N >= 64 && N % 64 == 0 && K >= kGemmChunk && K % kGemmChunk == 0 &&
           (int64_t)N * (K / 64) < ((int64_t)1 << 30) && (int64_t)M * K < ((int64_t)1 << 31) &&
           (int64_t)M * N < ((int64_t)1 << 40);
}

// Weight of the split partials in the automatic split choice: each extra
// split writes and re-reads M*N binary32 partials, 16*M/K of the weight bytes.
// Measured on MI355X with the 32x32x16 kernel (eight 32-column waves, OPT-175B
// projections, K = 12288): QKV (N = 36864, 144 column tiles) at M = 144:
// 233 / 184 / 206 / 194 us with 2..5 splits; output (N = 12288) at M = 144:
// 85 / 69 / 68 / 103 us with 3..6; at M = 32: QKV 90 / 73 / 79 / 75, output
// 36 / 31 / 31 / 42.  The weight 0.3 picks 3 and 5 at M = 144, 7 and 5 at M = 32.
constexpr double kGemmPartialWeight = 0.3;
constexpr int kGemmMaxAutoSplits = 16;

int gemm_splits(int M, int N, int K, int num_splits, int *chunks_per_split)
{
    const int chunks = K / kGemmChunk;
    int s = num_splits;
    if (s <= 0) {
        const int rows = 32 * kvq::gemm_row_blocks(M);
        const int64_t slots = kCUs;
        const int64_t tiles = (int64_t)((N + kGemmCols - 1) / kGemmCols) * ((M + rows - 1) / rows);
        const int max_s = std::max(1, chunks / 4); // at least 4 chunks per split
        // As many splits as one resident round holds ...
        s = (int)std::max<int64_t>(1, std::min<int64_t>(slots / std::max<int64_t>(tiles, 1), max_s));
        // ... unless that is one split of an under-filled round: then weigh the
        // rounds each split count needs against its partials.
        if (s == 1 && tiles < slots) {
            const double rho = 16.0 * M / K;
            double best = 1.0; // one split: one round, the whole K, no partials
            for (int c = 2; c <= std::min(max_s, kGemmMaxAutoSplits); ++c) {
                const int cps = (chunks + c - 1) / c;
                const int se = (chunks + cps - 1) / cps; // splits actually made
                const double rounds = std::ceil((double)(tiles * se) / (double)slots);
                const double cost = rounds * cps / chunks + kGemmPartialWeight * rho * se;
                if (cost < best - 1e-9) {
                    best = cost;
                    s = se;
                }
            }
        }
    }
    s = std::min(s, chunks);
    const int cps = (chunks + s - 1) / s;
    *chunks_per_split = cps;
    return (chunks + cps - 1) / cps; // no empty split
}

// The launch shape of one gemm_w4a16 call and the workspace it needs.
struct GemmPlan {
    int splits;        // 0: the stream form
    int chunks_per_split;
    int stream_groups; // workgroups of the stream form
    size_t ws_bytes;
};

// Stream form: one workgroup per CU, each over at least 4 (tile, chunk) units;
// its unit arithmetic is 32-bit (units x workgroups < 2^32).  Automatic choice:
// the split count above, unless its workgroups (tiles x splits) take more than
// one resident round -- then the stream form, which gives every CU the same
// number of units.  Measured on MI355X, OPT-175B projections (K = 12288) in
// decode-layer order (attention, QKV, output): QKV at M = 144 (3 splits, 432
// workgroups) 180.5 us split, 166.4 us stream; the output projection (5
// splits, 240 workgroups, one round) 68.8 us split, 79.3 us stream.
GemmPlan gemm_plan(int M, int N, int K, int num_splits)
{
    GemmPlan p{};
    const int rows = 32 * kvq::gemm_row_blocks(M);
    const int64_t tiles = (int64_t)((N + kGemmCols - 1) / kGemmCols) * ((M + rows - 1) / rows);
    const int64_t units = tiles * (K / kGemmChunk);
    const int64_t groups = std::min<int64_t>(kCUs, std::max<int64_t>(1, units / 4));
    const bool stream_ok = units * groups < ((int64_t)1 << 32);
    if (num_splits != KVQ_GEMM_STREAM) {
        p.splits = gemm_splits(M, N, K, num_splits, &p.chunks_per_split);
        p.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
        if (num_splits != 0 || tiles * p.splits <= kCUs || !stream_ok)
            return p;
    }
    if (!stream_ok) { // explicit stream form beyond its unit range
        p.splits = -1;
        return p;
    }
    p.splits = 0;
    p.chunks_per_split = 0;
    p.stream_groups = (int)groups;
    p.ws_bytes = (size_t)groups * 2 * (size_t)rows * kGemmCols * sizeof(float);
    return p;
}

bool gemm_splits_ok(int num_splits, int K)
{
    return num_splits == KVQ_GEMM_STREAM || (num_splits >= 0 && num_splits <= K / kGemmChunk);
}

} // namespace

extern "C" {

int kvq_cache_bytes(const kvq_dims *dims, size_t *codes_bytes_per_plane, size_t *meta_bytes_per_plane)
{
    int st = check_dims(dims);
    if (st != KVQ_OK)
        return st;
    const size_t slots = (size_t)dims->b * (size_t)dims->a * (size_t)(dims->s + dims->n);
    const size_t hd = (size_t)(dims->h / dims->a);
    if (codes_bytes_per_plane)
        *codes_bytes_per_plane = slots * hd / 2;
    if (meta_bytes_per_plane)
        *meta_bytes_per_plane = slots * (hd / KVQ_GROUP) * (dims->meta_dtype == KVQ_META_F16 ? 2 : 4);
    return KVQ_OK;
}

int kv_quantize_prefill(const kvq_cache *cache, const void *k_f16, const void *v_f16, int32_t s_len,
                        void *hip_stream)
{
    kvq::CachePlanes c;
    int st = check_cache(cache, &c);
    if (st != KVQ_OK)
        return st;
    if ((st = check_act(k_f16)) != KVQ_OK || (st = check_act(v_f16)) != KVQ_OK)
        return st;
    if (s_len < 1 || s_len > c.S)
        return KVQ_ERANGE;
    return status_of(kvq::launch_quantize(c, k_f16, v_f16, cache->dims.b, s_len, 0,
                                          static_cast<hipStream_t>(hip_stream)));
}

int kv_quantize_prefill_attend(const kvq_cache *cache, const void *q_f16, const void *k_f16, const void *v_f16,
                               int32_t s_len, void *out_f16, void *hip_stream)
{
    kvq::CachePlanes c;
    int st = check_cache(cache, &c);
    if (st != KVQ_OK)
        return st;
    if ((st = check_act(q_f16)) != KVQ_OK || (st = check_act(k_f16)) != KVQ_OK || (st = check_act(v_f16)) != KVQ_OK ||
        (st = check_act(out_f16)) != KVQ_OK)
        return st;
    if (s_len < 1 || s_len > c.S)
        return KVQ_ERANGE;
    // Byte offsets within one batch row's prompt (plus two tiles) must fit in 31 bits.
    if (((int64_t)s_len + 128) * cache->dims.h * 2 > 0x7FFFFFFF)
        return KVQ_EUNSUPPORTED;
    return status_of(kvq::launch_prefill(c, cache->dims.b, q_f16, k_f16, v_f16, s_len, out_f16,
                                         static_cast<hipStream_t>(hip_stream)));
}

int kv_append_quant(const kvq_cache *cache, const void *k_f16, const void *v_f16, int32_t pos, void *hip_stream)
{
    kvq::CachePlanes c;
    int st = check_cache(cache, &c);
    if (st != KVQ_OK)
        return st;
    if ((st = check_act(k_f16)) != KVQ_OK || (st = check_act(v_f16)) != KVQ_OK)
        return st;
    if (pos < 0 || pos >= c.S)
        return KVQ_ERANGE;
    return status_of(kvq::launch_quantize(c, k_f16, v_f16, cache->dims.b, 1, pos,
                                          static_cast<hipStream_t>(hip_stream)));
}

size_t kvq_workspace_bytes(const kvq_dims *dims, int32_t ctx_len, int32_t num_splits, int32_t k_top)
{
    if (check_dims(dims) != KVQ_OK)
        return 0;
    const int S = dims->s + dims->n;
    if (ctx_len < 1 || ctx_len > S || num_splits < 0 || num_splits > KVQ_MAX_SPLITS)
        return 0;
    const int pairs = dims->b * dims->a;
    if (k_top > 0)
        return ctx_len <= KVQ_TOPK_FUSED_MAX_CTX ? 0 : kvq::topk_ws_floats(pairs, ctx_len) * sizeof(float);
    const int hd = dims->h / dims->a;
    int len;
    const int s = resolve_splits(pairs, ctx_len, num_splits, &len);
    return kvq::decode_ws_floats(pairs, hd, s) * sizeof(float);
}

} // extern "C"

namespace {

// use_scratch: the split partials go to the library's static device
// workspace (decode_attention_q4_noalloc) instead of the caller's ws.
int decode_common(const kvq_cache *cache, const void *q_f16, int32_t ctx_len, void *out_f16, int32_t num_splits,
                  int32_t unroll, int32_t waves_per_pair, void *ws, size_t ws_bytes, const void *k_new,
                  const void *v_new, void *hip_stream, bool use_scratch = false)
{
    kvq::CachePlanes c;
    int st = check_cache(cache, &c);
    if (st != KVQ_OK)
        return st;
    if ((st = check_act(q_f16)) != KVQ_OK || (st = check_act(out_f16)) != KVQ_OK)
        return st;
    if (k_new != nullptr && ((st = check_act(k_new)) != KVQ_OK || (st = check_act(v_new)) != KVQ_OK))
        return st;
    if (ctx_len < 1 || ctx_len > c.S)
        return KVQ_ERANGE;
    if (num_splits < 0 || num_splits > KVQ_MAX_SPLITS)
        return KVQ_ERANGE;
    if ((unroll != 1 && unroll != 2 && unroll != 4) ||
        (waves_per_pair != kAutoWavesPerPair && waves_per_pair != 1 && waves_per_pair != 2 && waves_per_pair != 4))
        return KVQ_EINVAL;
    const int pairs = cache->dims.b * cache->dims.a;
    kvq::DecodeShape sh;
    sh.unroll = unroll;
    sh.splits = resolve_splits(pairs, ctx_len, num_splits, &sh.split_len);
    sh.waves_per_pair = waves_per_pair != kAutoWavesPerPair ? waves_per_pair
                        : (pairs < kFewPairs || (sh.splits == 1 && ctx_len >= kLongCtxFourWaves)) ? 4
                                                                                                 : kDefaultWavesPerPair;
    const size_t need = kvq::decode_ws_floats(pairs, c.d, sh.splits) * sizeof(float);
    if (use_scratch) {
        if (need > KVQ_NOALLOC_SCRATCH_BYTES)
            return KVQ_ENOSPACE;
        ws = nullptr;
        if (need > 0) {
            float *p = nullptr;
            if (kvq::noalloc_scratch(static_cast<hipStream_t>(hip_stream), &p) != 0)
                return KVQ_ELAUNCH;
            ws = p;
        }
    } else if (need > 0 && (ws == nullptr || !aligned16(ws) || ws_bytes < need)) {
        return ws_bytes < need ? KVQ_ENOSPACE : KVQ_EINVAL;
    }
    return status_of(kvq::launch_decode(c, pairs, q_f16, ctx_len, out_f16, sh, static_cast<float *>(ws), k_new,
                                        v_new, static_cast<hipStream_t>(hip_stream)));
}

} // namespace

extern "C" {

int decode_attention_q4_tuned(const kvq_cache *cache, const void *q_f16, int32_t ctx_len, void *out_f16,
                              int32_t num_splits, int32_t unroll, int32_t waves_per_pair, void *ws,
                              size_t ws_bytes, void *hip_stream)
{
    if (waves_per_pair == kAutoWavesPerPair)
        return KVQ_EINVAL; // the caller fixes the shape here
    return decode_common(cache, q_f16, ctx_len, out_f16, num_splits, unroll, waves_per_pair, ws, ws_bytes, nullptr,
                         nullptr, hip_stream);
}

int decode_attention_q4(const kvq_cache *cache, const void *q_f16, int32_t ctx_len, void *out_f16,
                        int32_t num_splits, void *ws, size_t ws_bytes, void *hip_stream)
{
    return decode_common(cache, q_f16, ctx_len, out_f16, num_splits, kDefaultUnroll, kAutoWavesPerPair, ws,
                         ws_bytes, nullptr, nullptr, hip_stream);
}

int decode_attention_q4_noalloc(const kvq_cache *cache, const void *q_f16, int32_t ctx_len, void *out_f16,
                                int32_t num_splits, void *hip_stream)
{
    return decode_common(cache, q_f16, ctx_len, out_f16, num_splits, kDefaultUnroll, kAutoWavesPerPair, nullptr, 0,
                         nullptr, nullptr, hip_stream, true);
}

int kv_append_attend_q4(const kvq_cache *cache, const void *q_f16, const void *k_f16, const void *v_f16,
                        int32_t pos, void *out_f16, int32_t num_splits, void *ws, size_t ws_bytes, void *hip_stream)
{
    if (k_f16 == nullptr || v_f16 == nullptr)
        return KVQ_EINVAL;
    if (cache != nullptr && check_dims(&cache->dims) == KVQ_OK && (pos < 0 || pos >= cache->dims.s + cache->dims.n))
        return KVQ_ERANGE;
    return decode_common(cache, q_f16, pos + 1, out_f16, num_splits, kDefaultUnroll, kAutoWavesPerPair, ws,
                         ws_bytes, k_f16, v_f16, hip_stream);
}

int decode_attention_q4_topk(const kvq_cache *cache, const void *q_f16, int32_t ctx_len, int32_t k_top,
                             void *out_f16, int32_t *sel_idx, void *ws, size_t ws_bytes, void *hip_stream)
{
    kvq::CachePlanes c;
    int st = check_cache(cache, &c);
    if (st != KVQ_OK)
        return st;
    if ((st = check_act(q_f16)) != KVQ_OK || (st = check_act(out_f16)) != KVQ_OK)
        return st;
    if (ctx_len < 1 || ctx_len > c.S)
        return KVQ_ERANGE;
    if (ctx_len > KVQ_TOPK_MAX_CTX)
        return KVQ_EUNSUPPORTED;
    if (k_top < 1 || k_top > ctx_len)
        return KVQ_ERANGE;
    if (sel_idx != nullptr && (reinterpret_cast<uintptr_t>(sel_idx) & 3u) != 0)
        return KVQ_EINVAL;
    const int pairs = cache->dims.b * cache->dims.a;
    const size_t need = kvq::topk_ws_floats(pairs, ctx_len) * sizeof(float);
    if (ws != nullptr || ctx_len > KVQ_TOPK_FUSED_MAX_CTX) { // scores kept in ws: it must hold them
        if (ws == nullptr || !aligned16(ws) || ws_bytes < need)
            return ws_bytes < need ? KVQ_ENOSPACE : KVQ_EINVAL;
    }
    return status_of(kvq::launch_topk(c, pairs, q_f16, ctx_len, k_top, out_f16, sel_idx, static_cast<float *>(ws),
                                      static_cast<hipStream_t>(hip_stream)));
}

int kvq_w4_quantize(const void *w_f16, int32_t N, int32_t K, uint8_t *codes, void *mins_f16, void *scales_f16,
                    void *hip_stream)
{
    if (!gemm_dims_ok(1, N, K))
        return KVQ_EINVAL;
    const void *ptrs[4] = {w_f16, codes, mins_f16, scales_f16};
    for (const void *p : ptrs)
        if (check_act(p) != KVQ_OK)
            return KVQ_EINVAL;
    return status_of(kvq::launch_quantize_weight(w_f16, N, K, codes, mins_f16, scales_f16,
                                                 static_cast<hipStream_t>(hip_stream)));
}

size_t kvq_gemm_w4_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t num_splits)
{
    if (!gemm_dims_ok(M, N, K) || !gemm_splits_ok(num_splits, K))
        return 0;
    const GemmPlan p = gemm_plan(M, N, K, num_splits);
    return p.splits < 0 ? 0 : p.ws_bytes;
}

int gemm_w4a16(const void *x_f16, int32_t M, int32_t N, int32_t K, const uint8_t *codes, const void *mins_f16,
               const void *scales_f16, void *y_f16, int32_t num_splits, void *ws, size_t ws_bytes,
               void *hip_stream)
{
    if (!gemm_dims_ok(M, N, K))
        return KVQ_EINVAL;
    const void *ptrs[5] = {x_f16, codes, mins_f16, scales_f16, y_f16};
    for (const void *p : ptrs)
        if (check_act(p) != KVQ_OK)
            return KVQ_EINVAL;
    if (!gemm_splits_ok(num_splits, K))
        return KVQ_ERANGE;
    const GemmPlan p = gemm_plan(M, N, K, num_splits);
    if (p.splits < 0)
        return KVQ_ERANGE;
    const size_t need = p.ws_bytes;
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return KVQ_ENOSPACE;
    if (need > 0 && !aligned16(ws))
        return KVQ_EINVAL;
    kvq::GemmArgs g{x_f16,   codes, mins_f16, scales_f16,         y_f16, static_cast<float *>(ws), M, N, K,
                    p.splits, p.chunks_per_split, p.stream_groups};
    return status_of(kvq::launch_gemm_w4(g, static_cast<hipStream_t>(hip_stream)));
}

int kv_quantize_prefill_host(const kvq_cache *cache, const void *k_f16, const void *v_f16, int32_t s_len,
                             int32_t n_threads)
{
    kvq::CachePlanes c;
    int st = check_cache(cache, &c);
    if (st != KVQ_OK)
        return st;
    if (k_f16 == nullptr || v_f16 == nullptr || n_threads < 0)
        return KVQ_EINVAL;
    if (s_len < 1 || s_len > c.S)
        return KVQ_ERANGE;
    return kvq::host_quantize(c, k_f16, v_f16, cache->dims.b, s_len, 0, n_threads) == 0 ? KVQ_OK : KVQ_ELAUNCH;
}

int kv_append_quant_host(const kvq_cache *cache, const void *k_f16, const void *v_f16, int32_t pos,
                         int32_t n_threads)
{
    kvq::CachePlanes c;
    int st = check_cache(cache, &c);
    if (st != KVQ_OK)
        return st;
    if (k_f16 == nullptr || v_f16 == nullptr || n_threads < 0)
        return KVQ_EINVAL;
    if (pos < 0 || pos >= c.S)
        return KVQ_ERANGE;
    return kvq::host_quantize(c, k_f16, v_f16, cache->dims.b, 1, pos, n_threads) == 0 ? KVQ_OK : KVQ_ELAUNCH;
}

int decode_attention_q4_host(const kvq_cache *cache, const void *q_f16, int32_t ctx_len, void *out_f16,
                             int32_t n_threads)
{
    kvq::CachePlanes c;
    int st = check_cache(cache, &c);
    if (st != KVQ_OK)
        return st;
    if (q_f16 == nullptr || out_f16 == nullptr || n_threads < 0)
        return KVQ_EINVAL;
    if (ctx_len < 1 || ctx_len > c.S)
        return KVQ_ERANGE;
    return kvq::host_attend(c, cache->dims.b * cache->dims.a, q_f16, ctx_len, out_f16, n_threads) == 0
               ? KVQ_OK
               : KVQ_ELAUNCH;
}

int kvq_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *hip_stream)
{
    if (check_act(buf) != KVQ_OK || sink == nullptr || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return KVQ_EINVAL;
    if (bytes < 16 || bytes % 16 != 0 || bytes / 16 / (256 * 16) >= 0x7FFFFFFF)
        return KVQ_ERANGE;
    return status_of(kvq::launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(hip_stream)));
}

int kvq_codec_params(const float *rng, int64_t n, int meta_dtype, float *scale, float *inv, void *hip_stream)
{
    if (n < 0 || n >= (int64_t)0x7FFFFFFF * 256)
        return KVQ_ERANGE;
    if (meta_dtype != KVQ_META_F32 && meta_dtype != KVQ_META_F16)
        return KVQ_EUNSUPPORTED;
    if (n == 0)
        return KVQ_OK;
    for (const void *p : {(const void *)rng, (const void *)scale, (const void *)inv})
        if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 3u) != 0)
            return KVQ_EINVAL;
    return status_of(kvq::launch_codec_params(rng, n, meta_dtype == KVQ_META_F16, scale, inv,
                                              static_cast<hipStream_t>(hip_stream)));
}

int kvq_host_simd() { return kvq::host_has_avx512(); }

void kvq_host_use_simd(int enable) { kvq::host_set_simd(enable); }

const char *kvq_strerror(int status)
{
    switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument (null or misaligned pointer, bad dimension)";
    case KVQ_ERANGE: return "argument out of range (s_len, pos, ctx_len, k_top or num_splits)";
    case KVQ_EUNSUPPORTED: return "unsupported configuration (group, metadata type, head_dim or context length)";
    case KVQ_ENOSPACE: return "workspace too small";
    case KVQ_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

} // extern "C"
