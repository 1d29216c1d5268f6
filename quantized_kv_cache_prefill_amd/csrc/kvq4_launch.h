// Internal interface between the C-ABI layer (kvq4_api.cpp) and the HIP
// kernels (kvq4_kernels.hip).  Arguments are already validated when these
// are called; each returns a hipError_t cast to int (0 = launched).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace kvq {

struct CachePlanes {
    uint8_t *k_codes, *v_codes;
    void *k_min, *k_scale, *v_min, *v_scale; // binary32, or binary16 when meta_f16
    int a;         // heads
    int d;         // head_dim (64, 128 or 256)
    int S;         // token slots per (batch row, head)
    bool meta_f16; // metadata planes hold binary16 values
};

// Quantise b*a*s_src token rows of fp16 K and V ([b][s_src][a][d]) into
// slots t_dst0 .. t_dst0+s_src-1.  Covers both the prompt (t_dst0 = 0) and
// the one-token append (s_src = 1, t_dst0 = pos).
int launch_quantize(const CachePlanes &c, const void *k, const void *v, int b, int s_src, int t_dst0,
                    hipStream_t st);

// Causal prefill attention over the prompt (fp16 q, k, v and out, each
// [b][s_len][a][d]) fused with the prompt's quantisation into slots
// 0..s_len-1 of the cache (the same planes launch_quantize writes).
int launch_prefill(const CachePlanes &c, int b, const void *q, const void *k, const void *v, int s_len, void *out,
                   hipStream_t st);

// Dense decode attention.  splits ranges of split_len tokens each; when
// splits > 1 the partial (max, sum, unnormalised output) go to ws and the
// reduce pass writes out.  With k_new/v_new non-null ([b][1][a][d] fp16),
// the same launch first quantises them into slot T-1 (fused append).
struct DecodeShape {
    int unroll;          // tokens per lane per iteration: 1, 2, 4
    int waves_per_pair;  // 1, 2, 4
    int splits;
    int split_len;
};
int launch_decode(const CachePlanes &c, int pairs, const void *q, int T, void *out, const DecodeShape &sh,
                  float *ws, const void *k_new, const void *v_new, hipStream_t st);

// Workspace floats needed by launch_decode for `splits` > 1.
size_t decode_ws_floats(int pairs, int d, int splits);

// Device address (on the device of stream st) of the library's static
// workspace of KVQ_NOALLOC_SCRATCH_BYTES; looked up once per device, never
// allocated.  Returns a hipError_t cast to int.
int noalloc_scratch(hipStream_t st, float **ptr);

// Top-k sparse decode attention: a streaming score pass into ws (one float
// per (pair, token)), then one workgroup per (batch row, head) for the
// selection and the gathered P.V.
int launch_topk(const CachePlanes &c, int pairs, const void *q, int T, int k_top, void *out, int32_t *sel,
                float *ws, hipStream_t st);

// Workspace floats needed by launch_topk.
size_t topk_ws_floats(int pairs, int T);

// y = x W^T with int4 weights (binary16 min/scale planes).  x fp16 [M][K],
// codes [N][K/2], mins/scales binary16 [N][K/64], y fp16 [M][N].  K % 128 == 0,
// N % 64 == 0.  splits > 1: binary32 partials in ws ([splits][M][N]) and a
// reduce pass.
struct GemmArgs {
    const void *x;
    const uint8_t *codes;
    const void *mins, *scales;
    void *y;
    float *ws;
    int M, N, K;
    int splits, chunks_per_split; // splits 0: the stream form over stream_groups workgroups
    int stream_groups;
};
int launch_gemm_w4(const GemmArgs &g, hipStream_t st);
int gemm_row_blocks(int M);

// Read `bytes` (a multiple of 16) of device memory once with the cache
// streams' load form; sink receives at most one word per 64 KB (normally
// none).
int launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st);

// The codec's stored scale and inverse scale (as binary32) for n group
// ranges rng[i] > 0, with binary32 (meta_f16 false) or binary16 metadata.
int launch_codec_params(const float *rng, int64_t n, bool meta_f16, float *scale, float *inv, hipStream_t st);

// Quantise W fp16 [N][K] with the binary16-metadata codec: codes [N][K/2],
// mins/scales binary16 [N][K/64].
int launch_quantize_weight(const void *w, int N, int K, uint8_t *codes, void *mins, void *scales, hipStream_t st);

// Host (CPU) path: the same planes and activations in host memory; work
// split over (batch row, head) pairs on n_threads threads (0 = all cores).
int host_quantize(const CachePlanes &c, const void *k, const void *v, int b, int s_src, int t_dst0, int n_threads);
int host_attend(const CachePlanes &c, int pairs, const void *q, int T, void *out, int n_threads);
int host_has_avx512();
void host_set_simd(int enable);

}  // namespace kvq
