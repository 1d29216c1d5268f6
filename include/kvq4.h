/*
 * kvq4.h -- int4 group-wise KV cache and decode-phase attention for MI355X
 * (gfx950).  C ABI: plain pointers and sizes only.
 *
 * What is computed, and where the pages define it:
 *
 *  - The KV cache of one transformer layer, prompt phase and decode phase:
 *    the FlexGen blog ("FlexGen: High-Throughput Generative Inference of
 *    Large Language Models with a Single GPU [ICML'23]", qingweiji blog),
 *    sections "预填充阶段" (prompt K/V of shape b x s x h) and "解码阶段"
 *    (each decode step concatenates the new token's K/V along the sequence
 *    axis, then attends with the single new query); section "KV Cache" gives
 *    the multi-head shape [b, s, a, h/a].  The notes on "A Survey on
 *    Efficient Inference for Large Language Models", section "Inference
 *    Process of LLMs", give the same prefill/decode split.
 *  - The cache is held compressed: "FlexGen研究学术报告" section 三.2(C)
 *    describes group-wise asymmetric 4-bit quantisation of the KV cache with
 *    64 contiguous elements per group, dequantised to FP16 before compute.
 *  - Attention scale 1/sqrt(d), d = h/a the per-head query/key dimension:
 *    the survey notes, eq. (2).
 *  - Sparse variant: the same report section, top-10% sparse attention
 *    (only the KV entries with the highest attention values are used).
 *
 * Readings taken where the pages are silent:
 *  - group axis = head_dim: group g of token row (b, t, a) is elements
 *    64g..64g+63 of that row; d must be a multiple of 64;
 *  - min/max affine code: scale = (max-min)/15, code = round_half_even(
 *    (x-min)*(15/(max-min))) clamped to 0..15, in binary32 with one rounding
 *    per operation; a constant group stores scale 0 and codes 0; a min of -0
 *    is stored as +0;
 *  - two codes per byte, the even element in the low nibble;
 *  - per-group min and scale kept as planes beside the codes, binary32
 *    (KVQ_META_F32) or binary16 (KVQ_META_F16).  With binary16 planes the
 *    min is stored exactly (it is one of the fp16 inputs), the scale is the
 *    binary32 quotient (max-min)/15 rounded to the nearest binary16 value
 *    (ties to even), and the codes are taken against that stored scale:
 *    code = round_half_even((x-min)*fl32(1/scale)) clamped to 0..15; a
 *    stored scale of 0 (constant group, or a scale that underflows binary16)
 *    gives codes 0.  Binary16 planes cut the cache from 160 to 144 bytes per
 *    (batch row, head, token) at d = 128.
 *
 * Device layout of one layer's cache (all planes caller-allocated):
 *    S = s + n token slots per (batch row, head);  G = d / 64
 *    k_codes, v_codes : uint8  [b][a][S][d/2]
 *    k_min, k_scale, v_min, v_scale : float32 or float16 [b][a][S][G]
 *  Slot t of (batch row bi, head ai) is row (bi*a + ai)*S + t.
 *  Activations passed in: fp16 (IEEE binary16), row-major, 16-byte aligned:
 *    prompt K/V      [b][s_len][a][d]
 *    q, new K/V, out [b][1][a][d]
 *
 * Conventions shared by every call:
 *  - Every pointer except the optional ones is a device pointer owned by
 *    the caller, who keeps it alive until the enqueued work has finished.
 *    Nothing here allocates, frees or synchronises: each call checks its
 *    arguments on the host, enqueues kernels on `hip_stream` (a
 *    hipStream_t; NULL = the default stream) and returns.  A kernel fault
 *    surfaces at the caller's next synchronisation.
 *  - Argument errors are reported before anything is enqueued, as a
 *    negative status; KVQ_OK (0) means the work was enqueued.
 *  - Inputs must be finite.  Overlapping calls that write the same cache
 *    slots race; calls on one stream are ordered.
 */
#ifndef KVQ4_H
#define KVQ4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    KVQ_OK = 0,
    KVQ_EINVAL = -1,        /* null or misaligned pointer, non-positive size, h % a != 0, d % 64 != 0 */
    KVQ_ERANGE = -2,        /* s_len, pos, ctx_len, k_top or num_splits outside its range            */
    KVQ_EUNSUPPORTED = -3,  /* group != 64, unknown metadata type, d not 64/128/256, context too long
                               ((s+n)*d/2 >= 2^31 for any call; see also the prefill and top-k limits) */
    KVQ_ENOSPACE = -4,      /* workspace smaller than kvq_workspace_bytes() asks for                 */
    KVQ_ELAUNCH = -5        /* the HIP runtime refused a launch                                      */
};

/* Metadata (min/scale) plane type. */
enum { KVQ_META_F32 = 0, KVQ_META_F16 = 1 };

#define KVQ_GROUP 64            /* elements per quantisation group                          */
#define KVQ_MAX_HEAD_DIM 256    /* d = h/a must be 64, 128 or 256                            */
#define KVQ_MAX_SPLITS 256      /* largest num_splits accepted by decode_attention_q4       */
#define KVQ_TOPK_MAX_CTX 8192   /* longest context decode_attention_q4_topk accepts        */
#define KVQ_TOPK_FUSED_MAX_CTX 2048 /* decode_attention_q4_topk up to this context: one launch */

/* Problem dimensions in the pages' notation: b batch (the effective batch of
 * one launch), a heads, h hidden size (d = h/a per head), s prompt length,
 * n generated tokens; the cache holds S = s + n slots ("P/D阶段计算" of the
 * FlexGen blog names b, s, n, h; "KV Cache" the multi-head shape
 * [b, s, a, h/a]).  Every call checks them: b, a, h, s > 0, n >= 0,
 * h % a == 0 and d % 64 == 0 (KVQ_EINVAL); group == 64, d in {64, 128, 256}
 * and a known meta_dtype (KVQ_EUNSUPPORTED); s + n <= 2^30 - 1 and
 * b * a <= 2^29 - 1 (KVQ_ERANGE); and S * d/2 < 2^31, since the tokens of one
 * (batch row, head) are addressed with 32-bit byte offsets (KVQ_EUNSUPPORTED:
 * at most 2^24 slots at d = 256, 2^25 at d = 128, 2^26 at d = 64). */
typedef struct kvq_dims {
    int32_t b, a, h, s, n;
    int32_t group;      /* must be KVQ_GROUP */
    int32_t meta_dtype; /* KVQ_META_F32 or KVQ_META_F16 */
} kvq_dims;

/* One layer's quantised cache: device pointers in the layout above. */
typedef struct kvq_cache {
    kvq_dims dims;
    uint8_t *k_codes, *v_codes;
    void *k_min, *k_scale, *v_min, *v_scale;
} kvq_cache;

/* Bytes of one code plane (k_codes or v_codes: b*a*S*d/2) and of one metadata
 * plane (each of k_min, k_scale, v_min, v_scale: b*a*S*(d/64)*4, or *2 for
 * KVQ_META_F16).  Either
 * output pointer may be NULL.  Host only; returns a status.
 * With precision 0.5 byte per element this is the blog's KV-cache size
 * 2*precision*layers*h*seq_len*batch (section "KV Cache") for one layer,
 * plus the metadata planes. */
int kvq_cache_bytes(const kvq_dims *dims, size_t *codes_bytes_per_plane, size_t *meta_bytes_per_plane);

/* Prompt phase: quantise the prompt's K and V (fp16 [b][s_len][a][d]) into
 * slots 0..s_len-1 of every (batch row, head).  1 <= s_len <= s+n.
 * Passage: the FlexGen blog, "预填充阶段" (the prompt's x_K, x_V of shape
 * b x s x h become the cache), with "FlexGen研究学术报告" 三.2(C) (the cache is
 * kept group-wise 4-bit, 64 contiguous elements per group). */
int kv_quantize_prefill(const kvq_cache *cache, const void *k_f16, const void *v_f16, int32_t s_len,
                        void *hip_stream);

/* Prompt phase with its attention, in one launch: writes exactly the planes
 * kv_quantize_prefill writes (slots 0..s_len-1, bit for bit) and
 * out = softmax(q k^T / sqrt(d)) v over the prompt, causal (row i over
 * tokens 0..i), for every (batch row, head).  The FlexGen blog's
 * "预填充阶段" gives x_out = softmax(x_Q x_K^T/sqrt(.)) x_V (before W_O and
 * the residual); causal because the decode step at position i sees tokens
 * 0..i; the attention reads the fp16 K and V (the int4 copy is for the
 * decode steps).  q, k, v, out: fp16 [b][s_len][a][d], device, 16-byte
 * aligned; out must not overlap q, k or v.  1 <= s_len <= s+n (KVQ_ERANGE);
 * (s_len + 128) * h * 2 bytes must be below 2^31 (KVQ_EUNSUPPORTED otherwise:
 * one batch row of the prompt is addressed with 32-bit offsets).
 * Accumulates in binary32 on the matrix cores; the probabilities enter the
 * P.V product as binary16. */
int kv_quantize_prefill_attend(const kvq_cache *cache, const void *q_f16, const void *k_f16, const void *v_f16,
                               int32_t s_len, void *out_f16, void *hip_stream);

/* Decode phase, KV update: quantise the new token's K and V (fp16
 * [b][1][a][d]) into slot `pos` of every (batch row, head), 0 <= pos < s+n.
 * Decode step j (1-based) appends at pos = s+j-1 and then attends over
 * ctx_len = s+j tokens.  Passage: the FlexGen blog, "解码阶段" (x_K <-
 * Concat(x_K, t W_K) along the sequence axis, the same for x_V), coded as in
 * "FlexGen研究学术报告" 三.2(C). */
int kv_append_quant(const kvq_cache *cache, const void *k_f16, const void *v_f16, int32_t pos,
                    void *hip_stream);

/* Workspace bytes decode_attention_q4 needs for (ctx_len, num_splits) -- 0
 * when the resolved split count is 1 -- or, when k_top > 0, the bytes
 * decode_attention_q4_topk needs: 0 for ctx_len <= KVQ_TOPK_FUSED_MAX_CTX,
 * else b*a*ctx_len*4 (one fp32 score per token).  Host only; returns 0 on
 * invalid arguments. */
size_t kvq_workspace_bytes(const kvq_dims *dims, int32_t ctx_len, int32_t num_splits, int32_t k_top);

/* Decode-phase attention over slots 0..ctx_len-1 (1 <= ctx_len <= s+n) of
 * every (batch row, head):
 *     out = softmax(q . K^T / sqrt(d)) . V      (per head; no W_O, no residual)
 * with K, V the dequantised cache.  q and out are fp16 [b][1][a][d].
 * Passage: the FlexGen blog, "解码阶段" (t_out = softmax(t_Q x_K^T/sqrt(.)) x_V
 * before W_O), with the 1/sqrt(d_k) of eq. (2) in the efficient-inference
 * survey notes and the cache dequantised per "FlexGen研究学术报告" 三.2(C).
 * Query elements that are binary16 subnormals (|q_i| < 2^-14) are taken as
 * 0: each score then differs from the exact one by at most
 * 2^-14 * sum_i |k_i| / sqrt(d) over those elements.
 * num_splits: 0 = choose automatically; k > 0 splits each context into at
 * most k ranges (when k > 1, each a whole number of 128-token blocks) handled
 * by separate workgroups and merged by a second pass (log-sum-exp).  ws: device workspace of ws_bytes >= kvq_workspace_bytes()
 * (may be NULL when that is 0). */
int decode_attention_q4(const kvq_cache *cache, const void *q_f16, int32_t ctx_len, void *out_f16,
                        int32_t num_splits, void *ws, size_t ws_bytes, void *hip_stream);

/* As decode_attention_q4 with the kernel's launch shape fixed by the caller:
 * unroll = tokens per lane per iteration (1, 2 or 4) and waves_per_pair =
 * waves sharing one (batch row, head) inside a workgroup (1, 2 or 4).
 * Results agree with decode_attention_q4 to rounding; for tuning and tests. */
int decode_attention_q4_tuned(const kvq_cache *cache, const void *q_f16, int32_t ctx_len, void *out_f16,
                              int32_t num_splits, int32_t unroll, int32_t waves_per_pair, void *ws,
                              size_t ws_bytes, void *hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * decode_attention_q4 with the split partials kept in a library-owned
 * static device array of KVQ_NOALLOC_SCRATCH_BYTES instead of a caller
 * workspace.  Same kernels, split choice and results as
 * decode_attention_q4(cache, q, ctx_len, out, num_splits, ...), bit for bit.
 * The call allocates and frees nothing; the array's device address is looked
 * up on the first call on each device (hipGetSymbolAddress) and each GPU
 * keeps its copy until the process ends.  KVQ_ENOSPACE (before anything is
 * enqueued) when the launch needs more than KVQ_NOALLOC_SCRATCH_BYTES, i.e.
 * kvq_workspace_bytes(dims, ctx_len, num_splits, 0) exceeds it: pass a
 * smaller num_splits.  KVQ_ELAUNCH when the address cannot be obtained.
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time (on different streams of one GPU) race and must be ordered by the
 * caller; calls on one stream are ordered. */
#define KVQ_NOALLOC_SCRATCH_BYTES (32u << 20)
int decode_attention_q4_noalloc(const kvq_cache *cache, const void *q_f16, int32_t ctx_len, void *out_f16,
                                int32_t num_splits, void *hip_stream);

/* One decode step in one launch: kv_append_quant(cache, k_new, v_new, pos)
 * followed by decode_attention_q4(cache, q, pos + 1, out, num_splits, ...),
 * the blog's "解码阶段" order (concatenate the new token's K/V, then attend
 * with its query).  0 <= pos < s+n; k_new, v_new, q, out fp16 [b][1][a][d];
 * the workspace is kvq_workspace_bytes(dims, pos + 1, num_splits, 0).
 * The cache planes and the output are bit-identical to the two separate
 * calls. */
int kv_append_attend_q4(const kvq_cache *cache, const void *q_f16, const void *k_f16, const void *v_f16,
                        int32_t pos, void *out_f16, int32_t num_splits, void *ws, size_t ws_bytes,
                        void *hip_stream);

/* Sparse decode attention: for every (batch row, head) score all ctx_len
 * tokens, keep the k_top highest scores (ties to the smaller token index),
 * and take the softmax and P.V over the kept tokens only.  Passage:
 * "FlexGen研究学术报告" 三.2(C), top-10% sparse attention (only the KV entries
 * with the highest attention values are loaded); scores as in
 * decode_attention_q4, subnormal query elements taken as 0 as there.
 * 1 <= k_top <= ctx_len <= min(s+n, KVQ_TOPK_MAX_CTX); the pages' rule keeps
 * k_top = ceil(0.1 * ctx_len).  sel_idx (device int32 [b][a][k_top], may be
 * NULL) receives the kept token indices in ascending order.
 * ws: the scores, fp32 [b][a][ctx_len] in log2 units (q . k * log2(e) /
 * sqrt(d)), the values the selection ranked.  Up to KVQ_TOPK_FUSED_MAX_CTX
 * tokens the call is one launch that keeps the scores on chip: ws may be NULL
 * (ws_bytes is then ignored), and a ws that is given receives the scores as
 * well, which costs that launch some 10%.  Longer contexts pass them between
 * two launches through ws, which is then required.  A ws that is given must
 * be 16-byte aligned with ws_bytes >= b*a*ctx_len*4 (KVQ_EINVAL, KVQ_ENOSPACE
 * otherwise). */
int decode_attention_q4_topk(const kvq_cache *cache, const void *q_f16, int32_t ctx_len, int32_t k_top,
                             void *out_f16, int32_t *sel_idx, void *ws, size_t ws_bytes, void *hip_stream);

/* ------------------------------------------------------------------------
 * Decode projections with int4 weights.  "FlexGen研究学术报告" section 三.2(C)
 * compresses the weights with the same group-wise asymmetric 4-bit code as
 * the KV cache and dequantises them to FP16 before compute; the FlexGen
 * blog's "解码阶段" applies them as t W_Q, t W_K, t W_V (and t_out W_O).
 * A weight W is given as in a linear layer, [N][K] fp16 (output row n,
 * input column k), and quantised row by row in groups of 64 contiguous k
 * with binary16 min/scale (the KVQ_META_F16 codec above).  The planes are
 * tiled so that each 64-row x 128-k block is contiguous:
 *    codes        : uint8   [N/64][K/128][64][64]  (row n%64, byte (k%128)/2,
 *                                                  even k in the low nibble)
 *    mins, scales : float16 [N/64][K/128][64][2]   (row n%64, group (k%128)/64)
 * The dequantised weight is the binary16 value nearest to min + code*scale
 * (sum exact, ties to even); y = x W^T accumulates in binary32 on the matrix
 * cores.  Requirements: N % 64 == 0, K % 128 == 0, N*K/64 < 2^30,
 * M*K < 2^31 (x is addressed with 32-bit byte offsets); every
 * pointer a 16-byte aligned device pointer owned by the caller.
 * ---------------------------------------------------------------------- */

/* Quantise W (fp16 [N][K]) into codes, mins and scales. */
int kvq_w4_quantize(const void *w_f16, int32_t N, int32_t K, uint8_t *codes, void *mins_f16, void *scales_f16,
                    void *hip_stream);

/* num_splits value of gemm_w4a16 that asks for the stream form: the
 * (output tile, 128-k chunk) units cut into one equal contiguous range per
 * compute unit, the tiles cut between ranges summed from binary32 partials by
 * a second pass.  Needs units x workgroups < 2^32 (KVQ_ERANGE otherwise);
 * the automatic choice takes it when the split form would need more than one
 * round of workgroups. */
#define KVQ_GEMM_STREAM (-1)

/* Workspace bytes gemm_w4a16 needs for num_splits (0 = automatic, chosen
 * from M, N, K only): binary32 partial sums [splits][M][N] when the K range
 * is split across workgroups, [workgroups][2][rows of a tile][256] in the
 * stream form, else 0. */
size_t kvq_gemm_w4_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t num_splits);

/* y (fp16 [M][N]) = x (fp16 [M][K]) times the transposed dequantised W, with
 * M >= 1 rows (the effective batch of one decode step).  num_splits: 0 =
 * automatic, KVQ_GEMM_STREAM = the stream form, else 1 <= num_splits <=
 * K/128 ranges of K (KVQ_ERANGE otherwise).  Every form gives the same y up
 * to the order of the binary32 sums.  ws: device workspace of ws_bytes >=
 * kvq_gemm_w4_workspace_bytes(M, N, K, num_splits) (may be NULL when that is
 * 0). */
int gemm_w4a16(const void *x_f16, int32_t M, int32_t N, int32_t K, const uint8_t *codes, const void *mins_f16,
               const void *scales_f16, void *y_f16, int32_t num_splits, void *ws, size_t ws_bytes,
               void *hip_stream);

/* ------------------------------------------------------------------------
 * Host path: the cache kept in CPU memory and the decode attention run on
 * the CPU, the placement "FlexGen研究学术报告" section 三.2(A) describes
 * (attention delegated to the CPU so the KV cache never crosses PCIe).  Same
 * operations, layout, codec and results as the GPU calls above, but every
 * pointer (the kvq_cache planes included) is HOST memory; the work is split
 * over (batch row, head) pairs on n_threads threads (0 = all cores) and the
 * call returns when it is done.  The codec and the attention use AVX-512
 * when the CPU has it (kvq_host_simd() returns 1), scalar loops otherwise;
 * both codecs give the same bits as the GPU's.  kvq_host_use_simd(0)
 * selects the scalar loops everywhere (process-wide, for comparison and
 * tests; not to be changed while another thread is inside a host call) and
 * kvq_host_use_simd(1) restores the default.  Errors: as the GPU calls
 * (KVQ_EINVAL for NULL pointers or bad dimensions, KVQ_ERANGE for s_len,
 * pos or ctx_len outside the cache); a cache plane that is device memory is
 * the caller's error and is not detected.
 * ---------------------------------------------------------------------- */
int kv_quantize_prefill_host(const kvq_cache *cache, const void *k_f16, const void *v_f16, int32_t s_len,
                             int32_t n_threads);
int kv_append_quant_host(const kvq_cache *cache, const void *k_f16, const void *v_f16, int32_t pos,
                         int32_t n_threads);
int decode_attention_q4_host(const kvq_cache *cache, const void *q_f16, int32_t ctx_len, void *out_f16,
                             int32_t n_threads);
int kvq_host_simd(void);
void kvq_host_use_simd(int enable);

/* ------------------------------------------------------------------------
 * Measurement: the HBM read ceiling the attention kernels are compared
 * with.  Decode attention is memory-bound (the efficient-inference survey
 * notes, "Efficiency Analysis": a very low compute-to-memory-access ratio),
 * so its roofline is the rate at which a kernel can stream memory.  This
 * call reads `bytes` of device memory at `buf` once, with the same 16-byte
 * nontemporal loads the cache streams use, and writes nothing but (almost
 * never) one word per 64 KB to `sink` (device, uint32 [ceil(bytes/65536)],
 * 4-byte aligned), which keeps the loads from being optimised away.  buf
 * 16-byte aligned; bytes a positive multiple of 16 (KVQ_ERANGE otherwise).
 * ---------------------------------------------------------------------- */
int kvq_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *hip_stream);

/* ------------------------------------------------------------------------
 * Verification: the codec's two divisions.  Every quantiser above stores
 * scale = (max - min)/15 and codes round((x - min) * inv) ("FlexGen研究学术报告"
 * section 三.2(C): group-wise asymmetric 4-bit, min/max affine code), with
 * binary32 metadata inv = 15/(max - min), with binary16 metadata scale
 * rounded to binary16 and inv = 1/scale; each quotient is meant to be the
 * correctly rounded binary32 value.  The kernels compute them without the
 * generic division sequence; this call runs that same device code on n
 * ranges rng[i] > 0 (device, binary32) and writes the stored scale (widened
 * to binary32) and the inverse to scale[i] and inv[i] (device, binary32), so
 * that every range the codec can meet can be checked.  meta_dtype
 * KVQ_META_F32 or KVQ_META_F16 (KVQ_EUNSUPPORTED otherwise); pointers
 * non-NULL and 4-byte aligned (KVQ_EINVAL); 0 <= n < 2^31 * 256
 * (KVQ_ERANGE).  Enqueued on hip_stream; nothing is allocated.
 * ---------------------------------------------------------------------- */
int kvq_codec_params(const float *rng, int64_t n, int meta_dtype, float *scale, float *inv, void *hip_stream);

/* Static text for a status code. */
const char *kvq_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ4_H */
