// Host (CPU) path over the same int4 cache layout held in host memory: the
// pages' alternative placement, where the compressed KV cache stays in CPU
// DRAM and the decode attention runs on the CPU so the cache never crosses
// PCIe ("FlexGen研究学术报告" section 三.2(A), delegating attention to the CPU;
// the same report's section 三.2(C) for the group-wise 4-bit code; the FlexGen
// blog's "解码阶段" for the decode step).
//
// Same operations and layout as the GPU calls: quantise the prompt's K/V into
// slots, append one token, and dense decode attention softmax(q K^T/sqrt(d)) V.
// The codec follows the binary32 (or binary16-metadata) definition step by
// step, so the planes are bit-identical to the GPU's; attention accumulates in
// binary32 with AVX-512 (when the CPU has it; a scalar loop otherwise), with
// the dequantisation folded out of the loops as on the GPU:
//   q.x = sum_g (scale_g * sum_{i in g} q_i c_i + min_g * sum_{i in g} q_i)
//   sum_t p_t x_t[i] = sum_t (p_t scale_g) c_t[i] + sum_t p_t min_g.
// Work is split over (batch row, head) pairs across n_threads std::threads.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>

#include <immintrin.h>

#include "kvq4_launch.h"

namespace kvq {
namespace {

constexpr int kGroup = 64;

inline float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
inline uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// ------------------------------------------------------------------ codec
// One group of 64 fp16 values: binary32, one rounding per operation, in the
// definition's order (min/max exact, -0 -> +0, rng = max - min; binary32
// metadata: scale = rng/15, inv = 15/rng; binary16 metadata: scale = the
// binary16 value nearest to rng/15, inv = 1/scale; code = clamp(rint((x -
// min) * inv), 0, 15), ties to even; a stored scale of 0 gives codes 0).
void quant_group(const uint16_t *x, uint8_t *codes, bool meta16, float *mn_out, float *sc_out)
{
#pragma clang fp contract(off)
    float f[kGroup];
    for (int i = 0; i < kGroup; ++i)
        f[i] = h2f(x[i]);
    float mn = f[0], mx = f[0];
    for (int i = 1; i < kGroup; ++i) {
        mn = f[i] < mn ? f[i] : mn;
        mx = f[i] > mx ? f[i] : mx;
    }
    mn = mn + 0.0f;
    mx = mx + 0.0f;
    const float rng = mx - mn;
    float scale = 0.0f, inv = 0.0f;
    if (!meta16) {
        if (rng != 0.0f) {
            scale = rng / 15.0f;
            inv = 15.0f / rng;
        }
    } else {
        if (rng != 0.0f)
            scale = h2f(f2h(rng / 15.0f));
        if (scale != 0.0f)
            inv = 1.0f / scale;
    }
    for (int j = 0; j < kGroup / 2; ++j) {
        int c[2] = {0, 0};
        if (scale != 0.0f) {
            for (int h = 0; h < 2; ++h) {
                float t = f[2 * j + h] - mn;
                t = t * inv;
                float r = rintf(t);
                r = r < 0.0f ? 0.0f : (r > 15.0f ? 15.0f : r);
                c[h] = (int)r;
            }
        }
        codes[j] = (uint8_t)(c[0] | (c[1] << 4));
    }
    *mn_out = mn;
    *sc_out = scale;
}

template <typename F>
void parallel_pairs(int pairs, int n_threads, F &&fn)
{
    int nt = n_threads > 0 ? n_threads : (int)std::max(1u, std::thread::hardware_concurrency());
    nt = std::max(1, std::min(nt, pairs));
    if (nt == 1) {
        fn(0, pairs);
        return;
    }
    std::vector<std::thread> th;
    th.reserve(nt);
    for (int i = 0; i < nt; ++i) {
        const int p0 = (int)((int64_t)pairs * i / nt), p1 = (int)((int64_t)pairs * (i + 1) / nt);
        th.emplace_back([&fn, p0, p1] { fn(p0, p1); });
    }
    for (auto &t : th)
        t.join();
}

// ------------------------------------------------------------ attention
// Metadata of token t, group g of one (batch row, head) stream, widened.
inline float meta_at(const void *plane, bool meta16, int64_t idx)
{
    return meta16 ? h2f(static_cast<const uint16_t *>(plane)[idx]) : static_cast<const float *>(plane)[idx];
}

// Scalar reference loop (any x86-64).
void attend_pair_scalar(const CachePlanes &c, int64_t pair, const uint16_t *q, int T, uint16_t *out)
{
    const int d = c.d, G = d / kGroup;
    const int64_t base = pair * c.S;
    const uint8_t *kc = c.k_codes + base * (d / 2), *vc = c.v_codes + base * (d / 2);
    std::vector<float> qf(d), acc(d, 0.0f), qsum(G, 0.0f), bsum(G, 0.0f);
    for (int i = 0; i < d; ++i) {
        qf[i] = h2f(q[i]);
        qsum[i / kGroup] += qf[i];
    }
    const float c2 = 1.0f / sqrtf((float)d);
    float m = -INFINITY, l = 0.0f;
    for (int t = 0; t < T; ++t) {
        const uint8_t *kr = kc + (int64_t)t * (d / 2);
        float s = 0.0f;
        for (int g = 0; g < G; ++g) {
            float dot = 0.0f;
            for (int i = 0; i < kGroup; ++i) {
                const int e = g * kGroup + i;
                const int code = (e & 1) ? (kr[e / 2] >> 4) : (kr[e / 2] & 15);
                dot += qf[e] * (float)code;
            }
            s += meta_at(c.k_scale, c.meta_f16, (base + t) * G + g) * dot +
                 meta_at(c.k_min, c.meta_f16, (base + t) * G + g) * qsum[g];
        }
        s *= c2;
        if (s > m) {
            const float alpha = expf(m - s);
            l *= alpha;
            for (int i = 0; i < d; ++i)
                acc[i] *= alpha;
            for (int g = 0; g < G; ++g)
                bsum[g] *= alpha;
            m = s;
        }
        const float p = expf(s - m);
        l += p;
        const uint8_t *vr = vc + (int64_t)t * (d / 2);
        for (int g = 0; g < G; ++g) {
            const float ps = p * meta_at(c.v_scale, c.meta_f16, (base + t) * G + g);
            bsum[g] += p * meta_at(c.v_min, c.meta_f16, (base + t) * G + g);
            for (int i = 0; i < kGroup; ++i) {
                const int e = g * kGroup + i;
                const int code = (e & 1) ? (vr[e / 2] >> 4) : (vr[e / 2] & 15);
                acc[e] += ps * (float)code;
            }
        }
    }
    for (int i = 0; i < d; ++i)
        out[i] = f2h((acc[i] + bsum[i / kGroup]) / l);
}

// AVX-512: a 32-element block of a row is 16 code bytes; the even elements
// (low nibbles) and odd elements (high nibbles) go to two zmm registers.
#define KVQ_AVX512 __attribute__((target("avx512f,avx512bw,avx512vl,avx512dq,f16c,fma")))

KVQ_AVX512 inline void unpack16(const uint8_t *p, __m512 &even, __m512 &odd)
{
    const __m512i b = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i *>(p)));
    even = _mm512_cvtepi32_ps(_mm512_and_si512(b, _mm512_set1_epi32(15)));
    odd = _mm512_cvtepi32_ps(_mm512_srli_epi32(b, 4));
}

// The codec of one group with 16-lane binary32 arithmetic: the same operations
// on the same values as quant_group (min and max are exact in any order; then
// x - min, times inv, round to nearest even, clamp), so the planes are
// bit-identical.  64 codes -> 64 bytes -> 32 words w; each word's two nibbles
// become one byte (w & 0xF) | ((w >> 4) & 0xF0).
KVQ_AVX512 inline __m128i codes16(__m512 f, __m512 vmn, __m512 vinv)
{
    __m512 t = _mm512_roundscale_ps(_mm512_mul_ps(_mm512_sub_ps(f, vmn), vinv),
                                    _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
    t = _mm512_min_ps(_mm512_max_ps(t, _mm512_setzero_ps()), _mm512_set1_ps(15.0f));
    return _mm512_cvtepi32_epi8(_mm512_cvttps_epi32(t));
}

KVQ_AVX512 void quant_group_avx512(const uint16_t *x, uint8_t *codes, bool meta16, float *mn_out, float *sc_out)
{
    __m512 f[4];
    for (int j = 0; j < 4; ++j)
        f[j] = _mm512_cvtph_ps(_mm256_loadu_si256(reinterpret_cast<const __m256i *>(x + 16 * j)));
    const float mn =
        _mm512_reduce_min_ps(_mm512_min_ps(_mm512_min_ps(f[0], f[1]), _mm512_min_ps(f[2], f[3]))) + 0.0f;
    const float mx =
        _mm512_reduce_max_ps(_mm512_max_ps(_mm512_max_ps(f[0], f[1]), _mm512_max_ps(f[2], f[3]))) + 0.0f;
    const float rng = mx - mn;
    float scale = 0.0f, inv = 0.0f;
    if (!meta16) {
        if (rng != 0.0f) {
            scale = rng / 15.0f;
            inv = 15.0f / rng;
        }
    } else {
        if (rng != 0.0f)
            scale = h2f(f2h(rng / 15.0f));
        if (scale != 0.0f)
            inv = 1.0f / scale;
    }
    __m256i packed = _mm256_setzero_si256();
    if (scale != 0.0f) {
        const __m512 vmn = _mm512_set1_ps(mn), vinv = _mm512_set1_ps(inv);
        __m512i b = _mm512_castsi128_si512(codes16(f[0], vmn, vinv));
        b = _mm512_inserti32x4(b, codes16(f[1], vmn, vinv), 1);
        b = _mm512_inserti32x4(b, codes16(f[2], vmn, vinv), 2);
        b = _mm512_inserti32x4(b, codes16(f[3], vmn, vinv), 3);
        const __m512i w = _mm512_or_si512(_mm512_and_si512(b, _mm512_set1_epi16(0x000F)),
                                          _mm512_and_si512(_mm512_srli_epi16(b, 4), _mm512_set1_epi16(0x00F0)));
        packed = _mm512_cvtepi16_epi8(w);
    }
    _mm256_storeu_si256(reinterpret_cast<__m256i *>(codes), packed);
    *mn_out = mn;
    *sc_out = scale;
}

// e^x for x <= 0, 16 lanes.  Cody-Waite range reduction x = n ln2 + f with
// |f| <= ln2/2 (ln 2 as a binary32 head and tail; the FMA keeps n*head exact),
// then e^f by its Taylor series to degree 7 (remainder below 1e-8 relative on
// that interval) and the factor 2^n by scalef.  Inputs below -104 give 0 or
// the smallest subnormal; -inf gives 0.
KVQ_AVX512 inline __m512 exp_neg_ps(__m512 x)
{
    x = _mm512_max_ps(x, _mm512_set1_ps(-104.0f));
    const __m512 n = _mm512_roundscale_ps(_mm512_mul_ps(x, _mm512_set1_ps(1.44269502f)),
                                          _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
    __m512 f = _mm512_fnmadd_ps(n, _mm512_set1_ps(0.693147182f), x);
    f = _mm512_fnmadd_ps(n, _mm512_set1_ps(-1.90465421e-09f), f);
    __m512 e = _mm512_set1_ps(1.0f / 5040.0f);
    e = _mm512_fmadd_ps(e, f, _mm512_set1_ps(1.0f / 720.0f));
    e = _mm512_fmadd_ps(e, f, _mm512_set1_ps(1.0f / 120.0f));
    e = _mm512_fmadd_ps(e, f, _mm512_set1_ps(1.0f / 24.0f));
    e = _mm512_fmadd_ps(e, f, _mm512_set1_ps(1.0f / 6.0f));
    e = _mm512_fmadd_ps(e, f, _mm512_set1_ps(0.5f));
    e = _mm512_fmadd_ps(e, f, _mm512_set1_ps(1.0f));
    e = _mm512_fmadd_ps(e, f, _mm512_set1_ps(1.0f));
    return _mm512_scalef_ps(e, n);
}

// Sixteen horizontal sums at once: out[t] = sum of the lanes of v[t].  Four
// halving steps (256-bit halves, 128-bit lanes, pairs, single lanes) leave
// token 4e + k in position 4k + e; the final permutation restores token order.
KVQ_AVX512 inline __m512 hsum16(const __m512 *v)
{
    __m512 r[8], u[4], w[2];
    for (int k = 0; k < 8; ++k)
        r[k] = _mm512_add_ps(_mm512_shuffle_f32x4(v[2 * k], v[2 * k + 1], 0x44),
                             _mm512_shuffle_f32x4(v[2 * k], v[2 * k + 1], 0xEE));
    for (int j = 0; j < 4; ++j)
        u[j] = _mm512_add_ps(_mm512_shuffle_f32x4(r[2 * j], r[2 * j + 1], 0x88),
                             _mm512_shuffle_f32x4(r[2 * j], r[2 * j + 1], 0xDD));
    for (int i = 0; i < 2; ++i)
        w[i] = _mm512_add_ps(_mm512_shuffle_ps(u[2 * i], u[2 * i + 1], _MM_SHUFFLE(1, 0, 1, 0)),
                             _mm512_shuffle_ps(u[2 * i], u[2 * i + 1], _MM_SHUFFLE(3, 2, 3, 2)));
    const __m512 x = _mm512_add_ps(_mm512_shuffle_ps(w[0], w[1], _MM_SHUFFLE(2, 0, 2, 0)),
                                   _mm512_shuffle_ps(w[0], w[1], _MM_SHUFFLE(3, 1, 3, 1)));
    const __m512i order = _mm512_setr_epi32(0, 4, 8, 12, 1, 5, 9, 13, 2, 6, 10, 14, 3, 7, 11, 15);
    return _mm512_permutexvar_ps(order, x);
}

// Blocks of 16 tokens: (1) the 16 scores, each token's K row reduced to one
// vector sum_g scale_g (q . c)_g and the 16 vectors summed horizontally in one
// pass; (2) the block's softmax update, one rescale of the accumulators per
// block; (3) the V rows folded into the accumulators with p_t scale_{t,g}.
template <int NB>
KVQ_AVX512 void attend_pair_avx512(const CachePlanes &c, int64_t pair, const uint16_t *q, int T, uint16_t *out)
{
    constexpr int d = 32 * NB, G = NB / 2, B = 16;
    const int64_t base = pair * c.S;
    const uint8_t *kc = c.k_codes + base * (d / 2), *vc = c.v_codes + base * (d / 2);
    alignas(64) float qf[d];
    for (int i = 0; i < d; ++i)
        qf[i] = h2f(q[i]);
    __m512 qe[NB], qo[NB];
    float qsum[G] = {};
    const __m512i idx_even = _mm512_setr_epi32(0, 2, 4, 6, 8, 10, 12, 14, 16, 18, 20, 22, 24, 26, 28, 30);
    const __m512i idx_odd = _mm512_add_epi32(idx_even, _mm512_set1_epi32(1));
    for (int j = 0; j < NB; ++j) {
        qe[j] = _mm512_i32gather_ps(idx_even, qf + 32 * j, 4);
        qo[j] = _mm512_i32gather_ps(idx_odd, qf + 32 * j, 4);
    }
    for (int i = 0; i < d; ++i)
        qsum[i / kGroup] += qf[i];
    __m512 ae[NB], ao[NB], bm[G];
    for (int j = 0; j < NB; ++j)
        ae[j] = ao[j] = _mm512_setzero_ps();
    for (int g = 0; g < G; ++g)
        bm[g] = _mm512_setzero_ps();
    const float c2 = 1.0f / sqrtf((float)d);
    float m = -INFINITY, l = 0.0f;
    alignas(64) __m512 red[B];
    alignas(64) float minterm[B], vsc[G][B], vmn[G][B], ps[G][B];
    for (int t0 = 0; t0 < T; t0 += B) {
        const int n = std::min(B, T - t0);
        for (int i = 0; i < B; ++i) {
            if (i >= n) {
                red[i] = _mm512_setzero_ps();
                minterm[i] = 0.0f;
                for (int g = 0; g < G; ++g)
                    vsc[g][i] = vmn[g][i] = 0.0f;
                continue;
            }
            const int64_t mi = (base + t0 + i) * G;
            const uint8_t *kr = kc + (int64_t)(t0 + i) * (d / 2);
            __m512 acc = _mm512_setzero_ps();
            float mt = 0.0f;
            for (int g = 0; g < G; ++g) {
                __m512 e0, o0, e1, o1;
                unpack16(kr + 32 * g, e0, o0);
                unpack16(kr + 32 * g + 16, e1, o1);
                __m512 dv = _mm512_mul_ps(qe[2 * g], e0);
                dv = _mm512_fmadd_ps(qo[2 * g], o0, dv);
                dv = _mm512_fmadd_ps(qe[2 * g + 1], e1, dv);
                dv = _mm512_fmadd_ps(qo[2 * g + 1], o1, dv);
                acc = _mm512_fmadd_ps(_mm512_set1_ps(meta_at(c.k_scale, c.meta_f16, mi + g)), dv, acc);
                mt += meta_at(c.k_min, c.meta_f16, mi + g) * qsum[g];
                vsc[g][i] = meta_at(c.v_scale, c.meta_f16, mi + g);
                vmn[g][i] = meta_at(c.v_min, c.meta_f16, mi + g);
            }
            red[i] = acc;
            minterm[i] = mt;
        }
        const __mmask16 live = (__mmask16)((1u << n) - 1u);
        __m512 sv = _mm512_mul_ps(_mm512_add_ps(hsum16(red), _mm512_load_ps(minterm)), _mm512_set1_ps(c2));
        sv = _mm512_mask_mov_ps(_mm512_set1_ps(-INFINITY), live, sv);
        const float m_new = std::max(m, _mm512_reduce_max_ps(sv));
        const __m512 p = _mm512_maskz_mov_ps(live, exp_neg_ps(_mm512_sub_ps(sv, _mm512_set1_ps(m_new))));
        if (m_new > m) {
            const float alpha = expf(m - m_new);
            const __m512 av = _mm512_set1_ps(alpha);
            l *= alpha;
            for (int j = 0; j < NB; ++j) {
                ae[j] = _mm512_mul_ps(ae[j], av);
                ao[j] = _mm512_mul_ps(ao[j], av);
            }
            for (int g = 0; g < G; ++g)
                bm[g] = _mm512_mul_ps(bm[g], av);
            m = m_new;
        }
        l += _mm512_reduce_add_ps(p);
        for (int g = 0; g < G; ++g) {
            _mm512_store_ps(ps[g], _mm512_mul_ps(p, _mm512_load_ps(vsc[g])));
            bm[g] = _mm512_fmadd_ps(p, _mm512_load_ps(vmn[g]), bm[g]);
        }
        for (int i = 0; i < n; ++i) {
            const uint8_t *vr = vc + (int64_t)(t0 + i) * (d / 2);
            for (int g = 0; g < G; ++g) {
                const __m512 pv = _mm512_set1_ps(ps[g][i]);
                __m512 e0, o0, e1, o1;
                unpack16(vr + 32 * g, e0, o0);
                unpack16(vr + 32 * g + 16, e1, o1);
                ae[2 * g] = _mm512_fmadd_ps(pv, e0, ae[2 * g]);
                ao[2 * g] = _mm512_fmadd_ps(pv, o0, ao[2 * g]);
                ae[2 * g + 1] = _mm512_fmadd_ps(pv, e1, ae[2 * g + 1]);
                ao[2 * g + 1] = _mm512_fmadd_ps(pv, o1, ao[2 * g + 1]);
            }
        }
    }
    alignas(64) float ev[16], ov[16];
    const float inv_l = 1.0f / l;
    for (int j = 0; j < NB; ++j) {
        _mm512_store_ps(ev, ae[j]);
        _mm512_store_ps(ov, ao[j]);
        const float b = _mm512_reduce_add_ps(bm[j / 2]);
        for (int i = 0; i < 16; ++i) {
            out[32 * j + 2 * i] = f2h((ev[i] + b) * inv_l);
            out[32 * j + 2 * i + 1] = f2h((ov[i] + b) * inv_l);
        }
    }
}

bool cpu_has_avx512()
{
    static const bool ok = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                           __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512dq") &&
                           __builtin_cpu_supports("f16c") && __builtin_cpu_supports("fma");
    return ok;
}

std::atomic<bool> g_simd_allowed{true}; // cleared by host_set_simd(0): the scalar loops even on AVX-512 CPUs

} // namespace

int host_quantize(const CachePlanes &c, const void *k, const void *v, int b, int s_src, int t_dst0, int n_threads)
{
    const int d = c.d, G = d / kGroup;
    const int pairs = b * c.a;
    const bool vec = g_simd_allowed && cpu_has_avx512();
    parallel_pairs(pairs, n_threads, [&](int p0, int p1) {
        for (int pair = p0; pair < p1; ++pair) {
            const int bi = pair / c.a, ai = pair % c.a;
            for (int which = 0; which < 2; ++which) {
                const uint16_t *src = static_cast<const uint16_t *>(which ? v : k);
                uint8_t *codes = which ? c.v_codes : c.k_codes;
                void *mins = which ? c.v_min : c.k_min;
                void *scales = which ? c.v_scale : c.k_scale;
                for (int ti = 0; ti < s_src; ++ti) {
                    const uint16_t *row = src + (((int64_t)bi * s_src + ti) * c.a + ai) * d;
                    const int64_t slot = (int64_t)pair * c.S + t_dst0 + ti;
                    for (int g = 0; g < G; ++g) {
                        float mn, sc;
                        uint8_t *cg = codes + slot * (d / 2) + g * (kGroup / 2);
                        if (vec)
                            quant_group_avx512(row + g * kGroup, cg, c.meta_f16, &mn, &sc);
                        else
                            quant_group(row + g * kGroup, cg, c.meta_f16, &mn, &sc);
                        if (c.meta_f16) {
                            static_cast<uint16_t *>(mins)[slot * G + g] = f2h(mn);
                            static_cast<uint16_t *>(scales)[slot * G + g] = f2h(sc);
                        } else {
                            static_cast<float *>(mins)[slot * G + g] = mn;
                            static_cast<float *>(scales)[slot * G + g] = sc;
                        }
                    }
                }
            }
        }
    });
    return 0;
}

int host_attend(const CachePlanes &c, int pairs, const void *q, int T, void *out, int n_threads)
{
    const bool vec = g_simd_allowed && cpu_has_avx512();
    const auto *qh = static_cast<const uint16_t *>(q);
    auto *oh = static_cast<uint16_t *>(out);
    parallel_pairs(pairs, n_threads, [&](int p0, int p1) {
        for (int pair = p0; pair < p1; ++pair) {
            const uint16_t *qp = qh + (int64_t)pair * c.d;
            uint16_t *op = oh + (int64_t)pair * c.d;
            if (vec && c.d == 64)
                attend_pair_avx512<2>(c, pair, qp, T, op);
            else if (vec && c.d == 128)
                attend_pair_avx512<4>(c, pair, qp, T, op);
            else if (vec && c.d == 256)
                attend_pair_avx512<8>(c, pair, qp, T, op);
            else
                attend_pair_scalar(c, pair, qp, T, op);
        }
    });
    return 0;
}

int host_has_avx512() { return g_simd_allowed && cpu_has_avx512() ? 1 : 0; }

void host_set_simd(int enable) { g_simd_allowed = enable != 0; }

} // namespace kvq
