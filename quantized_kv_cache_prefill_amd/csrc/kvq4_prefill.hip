// HIP kernel for gfx950: attention over the prompt (the prefill phase) fused
// with the prompt's quantisation into the int4 cache.
//
// Definitions followed (page titles and sections):
//  * prefill attention: the FlexGen blog, section "预填充阶段":
//    x_out = softmax(x_Q x_K^T / sqrt(.)) x_V, stopping before W_O and the
//    residual, with the per-head 1/sqrt(d_k) scale of eq. (2) in the
//    efficient-inference survey notes; causal (prompt token i attends to
//    tokens 0..i, the tokens the decode step at position i sees), over the
//    fp16 K and V as the projections produce them;
//  * the cache written beside it: "FlexGen研究学术报告" section 三.2(C),
//    group-wise asymmetric 4-bit, 64 contiguous elements per group -- the
//    same codec and planes as the prompt quantiser, bit for bit.
//
// Shape of the work.  Per (batch row, head) the attention is an s x s
// contraction over d, so it runs on the matrix cores
// (v_mfma_f32_16x16x32_f16, binary32 accumulation), flash-style: a
// workgroup owns 4 waves x 32 queries (16 per wave at d = 256) and walks the
// 64-key tiles up to its last query, keeping a running max and sum per query.
// Each wave computes S^T = K Q^T, so that the probabilities come out of the
// matrix core already in the operand layout of O^T = V^T P^T (the key index
// a lane holds is the same in both): only an fp32 -> fp16 conversion sits
// between the two products.  K and V tiles are staged through LDS
// (double-buffered, one barrier per tile): K row-major, V transposed at the
// write so that the V^T operand is two 8-byte reads.
//
// The fusion.  Every 64-key tile is read by all the query tiles at or after
// it; the workgroup whose queries cover that tile's positions (its diagonal)
// also runs the group codec on the fp16 rows it already holds in registers
// and writes their codes, mins and scales.  So each K/V row is quantised
// exactly once and the prompt is read from HBM once for both jobs.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvq4_device.h"
#include "kvq4_launch.h"

namespace kvq {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kKeys = 64;    // keys per K/V tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
struct Shape {
    static constexpr int QT = D <= 128 ? 2 : 1; // 16-query column tiles per wave
    static constexpr int QW = 16 * QT;          // queries per wave
    static constexpr int QB = kWaves * QW;      // queries per workgroup (128, or 64 at d = 256)
    static constexpr int KP = D + 8;            // K tile row pitch, halves (16-byte rows, offset banks)
    static constexpr int VP = kKeys + 8;        // V^T tile row pitch, halves
    static constexpr int KS = D / 32;           // k-steps of q.k
    static constexpr int DT = D / 16;           // 16-row tiles of O^T
    static constexpr int NK = kKeys * (D / 8) / kThreads;       // 16-byte K chunks per thread per tile
    static constexpr int NV = (kKeys / 2) * (D / 8) / kThreads; // V key pairs per thread per tile
    static constexpr int LDS_K = kKeys * KP;    // halves per K buffer
    static constexpr int LDS_V = D * VP;        // halves per V^T buffer
    static constexpr int LDS_HALVES = 2 * (LDS_K + LDS_V);
};

struct PrefillArgs {
    const uint16_t *q, *k, *v; // fp16 [b][s_len][a][D]
    uint16_t *out;             // fp16 [b][s_len][a][D]
    uint32_t *k_codes, *v_codes;
    void *k_min, *k_scale, *v_min, *v_scale;
    int a, S, s_len;
    int n_qtiles;   // query tiles per (batch row, head)
    int64_t total;  // pairs * n_qtiles
    int64_t chunk;  // work items per XCD slice
    float c2;       // log2(e) / sqrt(D)
};

// The prompt rows one thread moves per tile: NK 16-byte K chunks
// (key = id / (D/8), chunk c = id % (D/8), id = u*256 + tid) and NV pairs of
// V chunks (keys 2p and 2p+1 at the same chunk c).  Eight consecutive lanes
// hold the eight chunks of one 64-element group of one row, the layout the
// group codec needs.
template <int D>
struct TileRegs {
    uint4 k[Shape<D>::NK];
    uint4 v[2 * Shape<D>::NV];
};

__device__ __forceinline__ const uint4 *row_ptr(const uint16_t *base, int64_t bi, int tok, int a, int ai, int s_len,
                                                int D)
{
    return reinterpret_cast<const uint4 *>(base + (((bi * s_len + tok) * a + ai) * (int64_t)D));
}

template <int D>
__device__ __forceinline__ void load_tile(const PrefillArgs &g, int64_t bi, int ai, int j, TileRegs<D> &r)
{
    using Sh = Shape<D>;
    const int tid = threadIdx.x;
    const int c = tid % (D / 8);
#pragma unroll
    for (int u = 0; u < Sh::NK; ++u) {
        const int key = (u * kThreads + tid) / (D / 8);
        const int tok = min(kKeys * j + key, g.s_len - 1);
        r.k[u] = row_ptr(g.k, bi, tok, g.a, ai, g.s_len, D)[c];
    }
#pragma unroll
    for (int u = 0; u < Sh::NV; ++u) {
        const int p = (u * kThreads + tid) / (D / 8);
        const int t0 = min(kKeys * j + 2 * p, g.s_len - 1);
        const int t1 = min(kKeys * j + 2 * p + 1, g.s_len - 1);
        r.v[2 * u] = row_ptr(g.v, bi, t0, g.a, ai, g.s_len, D)[c];
        r.v[2 * u + 1] = row_ptr(g.v, bi, t1, g.a, ai, g.s_len, D)[c];
    }
}

template <typename Meta>
__device__ __forceinline__ void put_group(uint32_t *codes, Meta *mins, Meta *scales, int64_t slot, int D, int c,
                                          uint4 x, bool ok)
{
    uint32_t word;
    float mn, sc;
    quant_lane8<Meta>(x, word, mn, sc); // every lane of the wave takes part (DPP)
    if (ok) {
        __builtin_nontemporal_store(word, codes + slot * (D / 8) + c);
        if ((c & 7) == 0) {
            __builtin_nontemporal_store((Meta)mn, mins + slot * (D / 64) + (c >> 3));
            __builtin_nontemporal_store((Meta)sc, scales + slot * (D / 64) + (c >> 3));
        }
    }
}

// Write one tile to LDS (K row-major; V transposed: the two keys of a pair
// share one 32-bit word per element) and, on the diagonal, quantise its rows
// into the cache.
template <int D, typename Meta>
__device__ __forceinline__ void store_tile(const PrefillArgs &g, int64_t pair, int j, bool quantise,
                                           const TileRegs<D> &r, _Float16 *lk, _Float16 *lv)
{
    using Sh = Shape<D>;
    const int tid = threadIdx.x;
    const int c = tid % (D / 8);
#pragma unroll
    for (int u = 0; u < Sh::NK; ++u) {
        const int key = (u * kThreads + tid) / (D / 8);
        *reinterpret_cast<uint4 *>(lk + key * Sh::KP + 8 * c) = r.k[u];
    }
#pragma unroll
    for (int u = 0; u < Sh::NV; ++u) {
        const int p = (u * kThreads + tid) / (D / 8);
        const uint32_t a0[4] = {r.v[2 * u].x, r.v[2 * u].y, r.v[2 * u].z, r.v[2 * u].w};
        const uint32_t a1[4] = {r.v[2 * u + 1].x, r.v[2 * u + 1].y, r.v[2 * u + 1].z, r.v[2 * u + 1].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // element 2e: low halves of both keys; element 2e+1: high halves
            const uint32_t lo = __builtin_amdgcn_perm(a1[e], a0[e], 0x05040100u);
            const uint32_t hi = __builtin_amdgcn_perm(a1[e], a0[e], 0x07060302u);
            *reinterpret_cast<uint32_t *>(lv + (8 * c + 2 * e) * Sh::VP + 2 * p) = lo;
            *reinterpret_cast<uint32_t *>(lv + (8 * c + 2 * e + 1) * Sh::VP + 2 * p) = hi;
        }
    }
    if (quantise) {
        const int64_t base = pair * g.S;
#pragma unroll
        for (int u = 0; u < Sh::NK; ++u) {
            const int tok = kKeys * j + (u * kThreads + tid) / (D / 8);
            put_group<Meta>(g.k_codes, static_cast<Meta *>(g.k_min), static_cast<Meta *>(g.k_scale), base + tok, D,
                            c, r.k[u], tok < g.s_len);
        }
#pragma unroll
        for (int u = 0; u < Sh::NV; ++u) {
            const int tok = kKeys * j + 2 * ((u * kThreads + tid) / (D / 8));
            put_group<Meta>(g.v_codes, static_cast<Meta *>(g.v_min), static_cast<Meta *>(g.v_scale), base + tok, D,
                            c, r.v[2 * u], tok < g.s_len);
            put_group<Meta>(g.v_codes, static_cast<Meta *>(g.v_min), static_cast<Meta *>(g.v_scale), base + tok + 1,
                            D, c, r.v[2 * u + 1], tok + 1 < g.s_len);
        }
    }
}

template <int D, typename Meta>
__global__ __launch_bounds__(kThreads, 2) void k_prefill(PrefillArgs g)
{
    using Sh = Shape<D>;
    constexpr int QT = Sh::QT, KS = Sh::KS, DT = Sh::DT;
    __shared__ __attribute__((aligned(16))) _Float16 lds[Sh::LDS_HALVES];

    // Work item: the XCD this workgroup runs on (dispatch is round-robin over
    // the 8 XCDs) owns a contiguous slice of items, so the query tiles of one
    // (batch row, head) share that XCD's L2 for their K/V re-reads.  Within a
    // head the longest query tile (the last) comes first.
    const int64_t w = (int64_t)(blockIdx.x % 8) * g.chunk + blockIdx.x / 8;
    if (w >= g.total)
        return;
    const int64_t pair = w / g.n_qtiles;
    const int qtile = g.n_qtiles - 1 - (int)(w % g.n_qtiles);
    const int64_t bi = pair / g.a;
    const int ai = (int)(pair % g.a);
    const int q0 = qtile * Sh::QB;
    const int q_last = min(q0 + Sh::QB, g.s_len) - 1;
    const int n_tiles = q_last / kKeys + 1;
    const int j_diag = q0 / kKeys; // tiles j_diag.. hold this workgroup's own positions

    const int lane = threadIdx.x % 64;
    const int wave = threadIdx.x / 64;
    const int l16 = lane % 16, g4 = lane / 16;
    const int qw0 = q0 + wave * Sh::QW; // first query of this wave

    // Q^T operand: lane holds query qw0 + 16*qt + l16, d = 32*kd + 8*g4 .. +7.
    h8 qb[KS][QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int tok = min(qw0 + 16 * qt + l16, g.s_len - 1);
        const uint4 *row = row_ptr(g.q, bi, tok, g.a, ai, g.s_len, D);
#pragma unroll
        for (int kd = 0; kd < KS; ++kd)
            qb[kd][qt] = __builtin_bit_cast(h8, ld_stream16(row + 4 * kd + g4));
    }

    f4 o[DT][QT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
            o[t][qt] = f4{0.f, 0.f, 0.f, 0.f};
    float m[QT], l[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        m[qt] = -INFINITY;
        l[qt] = 0.f;
    }

    TileRegs<D> regs;
    load_tile<D>(g, bi, ai, 0, regs);
    store_tile<D, Meta>(g, pair, 0, 0 >= j_diag, regs, lds, lds + Sh::LDS_K);
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
        const bool more = j + 1 < n_tiles;
        if (more)
            load_tile<D>(g, bi, ai, j + 1, regs);
        const _Float16 *lk = lds + (j & 1) * (Sh::LDS_K + Sh::LDS_V);
        const _Float16 *lv = lk + Sh::LDS_K;
        if (kKeys * j <= qw0 + Sh::QW - 1) { // some key of the tile is visible to some query of the wave
            // S^T = K Q^T: st[c][qt] holds keys 16c + 4*g4 + r, query 16*qt + l16.
            f4 st[4][QT];
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int qt = 0; qt < QT; ++qt)
                    st[c][qt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kd = 0; kd < KS; ++kd) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const h8 ka = *reinterpret_cast<const h8 *>(lk + (16 * c + l16) * Sh::KP + 32 * kd + 8 * g4);
#pragma unroll
                    for (int qt = 0; qt < QT; ++qt)
                        st[c][qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[kd][qt], st[c][qt], 0, 0, 0);
                }
            }
            const bool masked = kKeys * j + kKeys - 1 > qw0;
            h8 pb[2][QT];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                const int qtok = qw0 + 16 * qt + l16;
                float mx = -INFINITY;
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float x = st[c][qt][r] * g.c2;
                        if (masked && kKeys * j + 16 * c + 4 * g4 + r > qtok)
                            x = -INFINITY;
                        st[c][qt][r] = x;
                        mx = fmaxf(mx, x);
                    }
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m[qt], mx);
                const float alpha = exp2_fast(m[qt] - m_new);
                m[qt] = m_new;
                float ls = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float p = exp2_fast(st[c][qt][r] - m_new);
                        st[c][qt][r] = p;
                        ls += p;
                    }
                l[qt] = l[qt] * alpha + ls;
#pragma unroll
                for (int t = 0; t < DT; ++t)
                    o[t][qt] *= alpha;
                // P^T operand of key step ks: slots 0..3 from key tile 2ks, 4..7 from 2ks+1.
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pb[ks][qt][r] = (_Float16)st[2 * ks][qt][r];
                        pb[ks][qt][4 + r] = (_Float16)st[2 * ks + 1][qt][r];
                    }
            }
            // O^T += V^T P^T: lane holds rows d = 16t + l16 of V^T at the same key slots.
#pragma unroll
            for (int t = 0; t < DT; ++t) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const _Float16 *vr = lv + (16 * t + l16) * Sh::VP + 32 * ks + 4 * g4;
                    const h4 v0 = *reinterpret_cast<const h4 *>(vr);
                    const h4 v1 = *reinterpret_cast<const h4 *>(vr + 16);
                    const h8 va = h8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
                    for (int qt = 0; qt < QT; ++qt)
                        o[t][qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[ks][qt], o[t][qt], 0, 0, 0);
                }
            }
        }
        if (more) {
            _Float16 *nk = lds + ((j + 1) & 1) * (Sh::LDS_K + Sh::LDS_V);
            store_tile<D, Meta>(g, pair, j + 1, j + 1 >= j_diag, regs, nk, nk + Sh::LDS_K);
        }
        __syncthreads();
    }

    // O = O^T / l: lane holds d = 16t + 4*g4 .. +3 of query 16*qt + l16.
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        float lt = l[qt];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const float inv = 1.0f / lt;
        const int qtok = qw0 + 16 * qt + l16;
        if (qtok < g.s_len) {
            uint16_t *row = g.out + (((bi * g.s_len + qtok) * g.a + ai) * (int64_t)D);
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const h4 h = h4{(_Float16)(o[t][qt][0] * inv), (_Float16)(o[t][qt][1] * inv),
                                (_Float16)(o[t][qt][2] * inv), (_Float16)(o[t][qt][3] * inv)};
                __builtin_nontemporal_store(__builtin_bit_cast(uint2, h).x,
                                            reinterpret_cast<uint32_t *>(row + 16 * t + 4 * g4));
                __builtin_nontemporal_store(__builtin_bit_cast(uint2, h).y,
                                            reinterpret_cast<uint32_t *>(row + 16 * t + 4 * g4) + 1);
            }
        }
    }
}

template <int D, typename Meta>
int launch_prefill_d(const CachePlanes &c, int b, const void *q, const void *k, const void *v, int s_len, void *out,
                     hipStream_t st)
{
    using Sh = Shape<D>;
    PrefillArgs g;
    g.q = static_cast<const uint16_t *>(q);
    g.k = static_cast<const uint16_t *>(k);
    g.v = static_cast<const uint16_t *>(v);
    g.out = static_cast<uint16_t *>(out);
    g.k_codes = reinterpret_cast<uint32_t *>(c.k_codes);
    g.v_codes = reinterpret_cast<uint32_t *>(c.v_codes);
    g.k_min = c.k_min;
    g.k_scale = c.k_scale;
    g.v_min = c.v_min;
    g.v_scale = c.v_scale;
    g.a = c.a;
    g.S = c.S;
    g.s_len = s_len;
    g.n_qtiles = (s_len + Sh::QB - 1) / Sh::QB;
    g.total = (int64_t)b * c.a * g.n_qtiles;
    g.chunk = (g.total + 7) / 8;
    g.c2 = kLog2e / sqrtf((float)D);
    const int64_t grid = 8 * g.chunk;
    if (grid > 0x7FFFFFFF)
        return (int)hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_prefill<D, Meta>), dim3((unsigned)grid), dim3(kThreads), 0, st, g);
    return (int)hipGetLastError();
}

template <typename Meta>
int launch_prefill_m(const CachePlanes &c, int b, const void *q, const void *k, const void *v, int s_len, void *out,
                     hipStream_t st)
{
    switch (c.d) {
    case 64: return launch_prefill_d<64, Meta>(c, b, q, k, v, s_len, out, st);
    case 128: return launch_prefill_d<128, Meta>(c, b, q, k, v, s_len, out, st);
    default: return launch_prefill_d<256, Meta>(c, b, q, k, v, s_len, out, st);
    }
}

} // namespace

int launch_prefill(const CachePlanes &c, int b, const void *q, const void *k, const void *v, int s_len, void *out,
                   hipStream_t st)
{
    return c.meta_f16 ? launch_prefill_m<_Float16>(c, b, q, k, v, s_len, out, st)
                      : launch_prefill_m<float>(c, b, q, k, v, s_len, out, st);
}

} // namespace kvq
