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
// between the two products.  K and V tiles go from HBM straight into LDS
// (gfx950's buffer loads to LDS: no staging registers, no LDS write
// instructions), double-buffered with one barrier per tile, both row-major
// with the 16-byte chunks of each row XOR-swizzled so that the operand reads
// hit distinct banks.  The V^T operand is read with the transposing LDS read
// (ds_read_b64_tr_b16: within each 16-lane group, lane i's element e comes
// from element i%4 of the 8 bytes lane 4e + i/4 addresses), so no transposed
// copy is ever written.
//
// The fusion.  Every 64-key tile is read by all the query tiles at or after
// it; the workgroup whose queries cover that tile's positions (its diagonal)
// also runs the group codec on the fp16 rows it already holds in LDS and
// writes their codes, mins and scales.  So each K/V row is quantised
// exactly once and the prompt is read from HBM once for both jobs.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "kvq4_device.h"
#include "kvq4_launch.h"

namespace kvq {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kKeys = 64;    // keys per K/V tile
constexpr int kWaves = 4;
constexpr int kPrefillCUs = 256; // one persistent workgroup per compute unit
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
struct Shape {
    static constexpr int QT = D <= 128 ? 2 : 1; // 16-query column tiles per wave
    static constexpr int QW = 16 * QT;          // queries per wave
    static constexpr int QB = kWaves * QW;      // queries per workgroup (128, or 64 at d = 256)
    static constexpr int KS = D / 32;           // k-steps of q.k
    static constexpr int DT = D / 16;           // 16-row tiles of O^T
    static constexpr int NK = kKeys * (D / 8) / kThreads; // 16-byte chunks per thread per tile, each of K and V
    static constexpr int LDS_K = kKeys * D;     // halves per K buffer (row pitch D)
    static constexpr int LDS_V = kKeys * D;     // halves per V buffer
    // Chunk swizzles: chunk c of row r sits at chunk c ^ swz(r) of that row.
    // RPW rows share one 256-byte bank window; NC chunks of a row are swizzled.
    static constexpr int RPW = D >= 128 ? 1 : 16 / (D / 8);
    static constexpr int NC = D / 8 < 16 ? D / 8 : 16;
    // K: 16-byte reads of 16 consecutive rows at one chunk land in 16 distinct
    // 16-byte bank groups.
    static __device__ __forceinline__ int swz_k(int r) { return (r / RPW) % NC; }
    // V: 8-byte transposing reads of 4 consecutive rows x 2 chunks land in 8
    // distinct bank groups (even swizzle, so a chunk pair stays a pair).
    static __device__ __forceinline__ int swz_v(int r) { return 2 * ((r / RPW) % (NC / 2)); }
    static constexpr int LDS_HALVES = 2 * (LDS_K + LDS_V);
};

struct PrefillArgs {
    const uint16_t *q, *k, *v; // fp16 [b_chunk][s_len][a][D], this launch's batch rows
    uint16_t *out;             // fp16 [b_chunk][s_len][a][D]
    uint32_t *k_codes, *v_codes;
    void *k_min, *k_scale, *v_min, *v_scale;
    int64_t pair0;  // cache (batch row, head) index of this launch's first pair
    int bytes;      // bytes of each of q, k, v in this launch (< 2^31)
    int a, S, s_len;
    int n_qtiles;   // query tiles per (batch row, head)
    int64_t total;  // pairs * n_qtiles
    int64_t chunk;  // work items per XCD slice
    float c2;       // log2(e) / sqrt(D)
    float slack;    // raw-score growth allowed before the accumulators are rescaled: 8 / c2
};

// The prompt tensors are read through buffer resources whose size is the
// launch's bytes of q, k or v.  Every offset, the key-tile step included, is
// passed in the lane's 32-bit VGPR offset: the hardware range check covers
// that offset (not the scalar offset), so a read at or past the end of the
// tensor returns zeros instead of the memory behind it.  That happens for
// the rows of the last key tile past the prompt in the launch's last batch
// row; those keys are masked (p = 0), and zeros keep 0 * V finite.
typedef uint32_t u32x4b __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
// 16 bytes per lane, HBM -> LDS: lane l's bytes land at dst + 16 l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, _Float16 *dst, int voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

// One tile of K and V, HBM -> LDS.  Wave w's u-th load fills 1 KB block
// B = 4u + w of each buffer: lane l writes chunk position 64B + l, i.e. row
// (64B + l) / (D/8), swizzled chunk (64B + l) % (D/8); vk/vv hold the byte
// offsets (tile 0) of the unswizzled chunks that belong there, `step` the
// byte offset of this tile.
template <int D>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, const int *vk,
                                           const int *vv, int step, _Float16 *lk, _Float16 *lv, int wave)
{
#pragma unroll
    for (int u = 0; u < Shape<D>::NK; ++u) {
        const int blk = 4 * u + wave;
        dma16(rk, lk + 512 * blk, vk[u] + step);
        dma16(rv, lv + 512 * blk, vv[u] + step);
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

// The codes of 8 consecutive fp16 values against a group's stored min and
// inverse scale, element i at bits 4i..4i+3 (the code step of quant_lane8).
template <typename Meta>
__device__ __forceinline__ uint32_t codes8(const uint4 x, float mn, float inv)
{
#pragma clang fp contract(off)
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t ev = 0, od = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float te = sub_lo16(w[j], mn) * inv;
        float to = sub_hi16(w[j], mn) * inv;
        if constexpr (sizeof(Meta) != 4) {
            te = fminf(te, 15.0f);
            to = fminf(to, 15.0f);
        }
        ev = __builtin_amdgcn_cvt_pk_u8_f32(te, j, ev);
        od = __builtin_amdgcn_cvt_pk_u8_f32(to, j, od);
    }
    return ev | (od << 4);
}

// The same codec for one lane's 16 consecutive fp16 values (x0: elements
// 0..7, x1: 8..15); 4 consecutive lanes (an aligned quad) hold one
// 64-element group, so the group reduction takes two cross-lane steps and the
// stored min and scale are formed once per 16 elements.  Same arithmetic,
// same results as quant_lane8 on the group.
template <typename Meta>
__device__ __forceinline__ void quant_lane16(const uint4 x0, const uint4 x1, uint32_t &w0, uint32_t &w1, float &mn_out,
                                             float &scale_out)
{
#pragma clang fp contract(off)
    const uint32_t lo = pk_min16(pk_min16(pk_min16(x0.x, x0.y), pk_min16(x0.z, x0.w)),
                                 pk_min16(pk_min16(x1.x, x1.y), pk_min16(x1.z, x1.w)));
    const uint32_t hi = pk_max16(pk_max16(pk_max16(x0.x, x0.y), pk_max16(x0.z, x0.w)),
                                 pk_max16(pk_max16(x1.x, x1.y), pk_max16(x1.z, x1.w)));
    uint32_t p = pk_min_neg_hi(lo, hi);
    p = pk_min16(p, dpp_u<kQuadXor1>(p));
    p = pk_min16(p, dpp_u<kQuadXor2>(p));
    const float mn = h2f_lo(p) + 0.0f; // -0 -> +0
    const float mx = -h2f_hi(p) + 0.0f;
    float scale, inv;
    codec_params<Meta>(mx - mn, scale, inv);
    w0 = codes8<Meta>(x0, mn, inv);
    w1 = codes8<Meta>(x1, mn, inv);
    mn_out = mn;
    scale_out = scale;
}


// head_dim 128: one lane's 16-element piece of a token row (elements 16cc ..
// 16cc + 15, cc = 0..7), quantised by quant_lane16, and its stores with the
// plane bases of one (batch row, head) (uniform) and the token's index within
// it: 32-bit offsets only.
struct QPiece {
    uint32_t w0, w1; // codes of elements 16cc .. 16cc + 7 and 16cc + 8 .. 16cc + 15
    float mn, sc;    // the group's stored min and scale
};
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <typename Meta>
__device__ __forceinline__ void put_piece(uint32_t *codes, Meta *mins, Meta *scales, int tok, int cc, const QPiece &q)
{
    __builtin_nontemporal_store(u32x2{q.w0, q.w1}, reinterpret_cast<u32x2 *>(codes + (uint32_t)(tok * 16 + 2 * cc)));
    if ((cc & 3) == 0) {
        __builtin_nontemporal_store((Meta)q.mn, mins + (uint32_t)(tok * 2 + (cc >> 2)));
        __builtin_nontemporal_store((Meta)q.sc, scales + (uint32_t)(tok * 2 + (cc >> 2)));
    }
}

// Quantise the rows of one tile (this workgroup's diagonal) into the cache,
// reading them back from LDS: thread chunk (key (u*256 + tid) / (D/8), chunk
// tid % (D/8)), eight consecutive lanes per 64-element group.
template <int D, typename Meta>
__device__ __forceinline__ void quantise_tile(const PrefillArgs &g, int64_t pair, int j, const _Float16 *lk,
                                              const _Float16 *lv)
{
    using Sh = Shape<D>;
    const int tid = threadIdx.x;
    const int c = tid % (D / 8);
    const int64_t base = pair * g.S;
#pragma unroll
    for (int u = 0; u < Sh::NK; ++u) {
        const int key = (u * kThreads + tid) / (D / 8);
        const int tok = kKeys * j + key;
        const uint4 xk = *reinterpret_cast<const uint4 *>(lk + key * D + 8 * (c ^ Sh::swz_k(key)));
        const uint4 xv = *reinterpret_cast<const uint4 *>(lv + key * D + 8 * (c ^ Sh::swz_v(key)));
        put_group<Meta>(g.k_codes, static_cast<Meta *>(g.k_min), static_cast<Meta *>(g.k_scale), base + tok, D, c,
                        xk, tok < g.s_len);
        put_group<Meta>(g.v_codes, static_cast<Meta *>(g.v_min), static_cast<Meta *>(g.v_scale), base + tok, D, c,
                        xv, tok < g.s_len);
    }
}

// Lane l and lane l ^ 16 (l ^ 32) combined, through the gfx950 lane swaps
// instead of an LDS permute: with both operands a copy of x, v_permlane16_swap
// leaves rows (0, 0, 2, 2) of x in one result and rows (1, 1, 3, 3) in the
// other (v_permlane32_swap: halves (lo, lo) and (hi, hi)), so every lane holds
// its own value and its partner's, in the same order in both lanes.
template <bool ADD>
__device__ __forceinline__ float xor_lanes16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                    false, false);
    const float a = __builtin_bit_cast(float, (uint32_t)r[0]), b = __builtin_bit_cast(float, (uint32_t)r[1]);
    return ADD ? a + b : fmaxf(a, b);
}
template <bool ADD>
__device__ __forceinline__ float xor_lanes32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                    false, false);
    const float a = __builtin_bit_cast(float, (uint32_t)r[0]), b = __builtin_bit_cast(float, (uint32_t)r[1]);
    return ADD ? a + b : fmaxf(a, b);
}

// 8 bytes through the transposing LDS read.
typedef short s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4 lds_s4;
__device__ __forceinline__ h4 ld_tr(const _Float16 *p)
{
    return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(p)));
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
    const int64_t lpair = w / g.n_qtiles; // pair within this launch
    const int qtile = g.n_qtiles - 1 - (int)(w % g.n_qtiles);
    const int bi = (int)(lpair / g.a);
    const int ai = (int)(lpair % g.a);
    const int64_t pair = g.pair0 + lpair;
    const int q0 = qtile * Sh::QB;
    const int q_last = min(q0 + Sh::QB, g.s_len) - 1;
    const int n_tiles = q_last / kKeys + 1;
    const int j_diag = q0 / kKeys; // tiles j_diag.. hold this workgroup's own positions

    const int lane = threadIdx.x % 64;
    const int wave = threadIdx.x / 64;
    const int l16 = lane % 16, g4 = lane / 16;
    const int qw0 = q0 + wave * Sh::QW; // first query of this wave

    const int row_bytes = g.a * D * 2;                 // one token row of all heads
    const int head0 = (bi * g.s_len * g.a + ai) * D * 2; // token 0 of this (batch row, head)
    const __amdgpu_buffer_rsrc_t rq = rsrc(g.q, g.bytes), rk = rsrc(g.k, g.bytes), rv = rsrc(g.v, g.bytes);

    // The workgroup's QB query rows go HBM -> LDS (the second tile buffer, free until
    // the loop fills it) as whole rows, chunks swizzled as K's (queries past the
    // prompt read the next rows or zeros; their outputs are not stored).
    {
        constexpr int NQ = Sh::QB * (D / 8) / kThreads;
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            const int blk = 4 * u + wave;
            const int pos = 64 * blk + lane;
            const int r = pos / (D / 8), cs = pos % (D / 8);
            dma16(rq, lds + Sh::LDS_K + Sh::LDS_V + 512 * blk, head0 + (q0 + r) * row_bytes + 16 * (cs ^ Sh::swz_k(r)));
        }
    }
    // Byte offsets (tile 0) of the chunks this lane moves into LDS.
    int vk[Sh::NK], vv[Sh::NK];
#pragma unroll
    for (int u = 0; u < Sh::NK; ++u) {
        const int pos = 64 * (4 * u + wave) + lane;
        const int r = pos / (D / 8), cs = pos % (D / 8);
        vk[u] = head0 + r * row_bytes + 16 * (cs ^ Sh::swz_k(r));
        vv[u] = head0 + r * row_bytes + 16 * (cs ^ Sh::swz_v(r));
    }
    const int tile_bytes = kKeys * row_bytes;

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

    issue_tile<D>(rk, rv, vk, vv, 0, lds, lds + Sh::LDS_K, wave);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // Q^T operand: lane holds query qw0 + 16*qt + l16, d = 32*kd + 8*g4 .. +7.
    h8 qb[KS][QT];
    {
        const _Float16 *lq = lds + Sh::LDS_K + Sh::LDS_V;
        const int sq = Sh::swz_k(l16); // query rows 16m + l16 all share it
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int kd = 0; kd < KS; ++kd)
                qb[kd][qt] = *reinterpret_cast<const h8 *>(lq + (wave * Sh::QW + 16 * qt + l16) * D +
                                                           8 * ((4 * kd + g4) ^ sq));
    }
    __syncthreads(); // the query rows are in registers before tile 1 overwrites them

    for (int j = 0; j < n_tiles; ++j) {
        const bool more = j + 1 < n_tiles;
        if (more) { // into the other buffer, which every wave finished reading before the last barrier
            _Float16 *nk = lds + ((j + 1) & 1) * (Sh::LDS_K + Sh::LDS_V);
            issue_tile<D>(rk, rv, vk, vv, (j + 1) * tile_bytes, nk, nk + Sh::LDS_K, wave);
        }
        const _Float16 *lk = lds + (j & 1) * (Sh::LDS_K + Sh::LDS_V);
        const _Float16 *lv = lk + Sh::LDS_K;
        if (kKeys * j <= qw0 + Sh::QW - 1) { // some key of the tile is visible to some query of the wave
            // S^T = K Q^T: st[c][qt] holds keys 16c + 4*g4 + r, query 16*qt + l16.  The K
            // operands of step kd+1 are read from LDS while the products of step kd run.
            f4 st[4][QT];
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int qt = 0; qt < QT; ++qt)
                    st[c][qt] = f4{0.f, 0.f, 0.f, 0.f};
            // Steps (kd, c) in order; the K operand of step i+3 is read while the
            // products of step i run (a ring of four operands).
            constexpr int NS = KS * 4, LA = 3;
            const int sk = Sh::swz_k(l16); // rows 16c + l16 all share it
            auto ld_ka = [&](int n) {
                return *reinterpret_cast<const h8 *>(lk + (16 * (n % 4) + l16) * D + 8 * ((4 * (n / 4) + g4) ^ sk));
            };
            h8 ka[4];
#pragma unroll
            for (int i = 0; i < LA; ++i)
                ka[i] = ld_ka(i);
            // The first LA reads form a group of their own, ahead of the (read,
            // products) groups: without it the scheduler fills those groups' read
            // slots with them and every product waits on the read just before it.
            __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int kd = i / 4, c = i % 4;
                if (i + LA < NS)
                    ka[(i + LA) % 4] = ld_ka(i + LA);
#pragma unroll
                for (int qt = 0; qt < QT; ++qt)
                    st[c][qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[i % 4], qb[kd][qt], st[c][qt], 0, 0, 0);
                if (i + LA < NS) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // a later step's LDS read,
                    __builtin_amdgcn_sched_group_barrier(0x008, QT, 0); // then this step's products
                }
            }
            // Online softmax on the raw scores (the scale c2 > 0 is applied inside the
            // exponent), both query tiles side by side so their cross-lane steps overlap.
            // Keys after a query are masked only in the diagonal tiles.
            if (kKeys * j + kKeys - 1 > qw0) {
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) {
                    const int rel = qw0 + 16 * qt + l16 - kKeys * j - 4 * g4; // key offset limit
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (16 * c + r > rel)
                                st[c][qt][r] = -INFINITY;
                }
            }
            float mx[QT];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                mx[qt] = st[0][qt][0];
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        mx[qt] = fmaxf(mx[qt], st[c][qt][r]);
            }
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
                mx[qt] = xor_lanes16<false>(mx[qt]);
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
                mx[qt] = xor_lanes32<false>(mx[qt]);
            // The reference m only moves when some query's max exceeds it by more than
            // 8 (log2 units): probabilities up to 2^8 are exact enough in fp16 and the
            // sum and accumulators are binary32, so the result is the same softmax with
            // far fewer rescales of O.
            bool grow = false;
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
                grow |= mx[qt] > m[qt] + g.slack;
            if (__any(grow)) {
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) {
                    const float m_new = fmaxf(m[qt], mx[qt]);
                    const float alpha = exp2_fast((m[qt] - m_new) * g.c2);
                    m[qt] = m_new;
                    l[qt] *= alpha;
#pragma unroll
                    for (int t = 0; t < DT; ++t)
                        o[t][qt] *= alpha;
                }
            }
            h8 pb[2][QT];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                const float mb = -m[qt] * g.c2;
                float ls = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float p = exp2_fast(__builtin_fmaf(st[c][qt][r], g.c2, mb));
                        st[c][qt][r] = p;
                        ls += p;
                    }
                l[qt] += ls;
                // P^T operand of key step ks: slots 0..3 from key tile 2ks, 4..7 from 2ks+1.
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pb[ks][qt][r] = (_Float16)st[2 * ks][qt][r];
                        pb[ks][qt][4 + r] = (_Float16)st[2 * ks + 1][qt][r];
                    }
            }
            // O^T += V^T P^T.  The A operand of row tile t, key step ks: lane (l16, g4) holds
            // V[key][16t + l16] for keys 32ks + 4*g4 + (0..3) and 32ks + 16 + 4*g4 + (0..3).
            // Transposing reads: lane (i, g4) addresses row 32ks + 4*g4 + i/4 (and +16),
            // columns 16t + 4*(i%4) .. +3, i.e. chunk 2t + (i%4)/2, half i%2 of it.
            const int vrow = 4 * g4 + l16 / 4;
            const int sv = Sh::swz_v(vrow); // the same for rows vrow + 16k
            const _Float16 *vbase = lv + vrow * D + 4 * (l16 % 2);
            // Steps (t, ks) in order, the operand of step i+3 read during step i.
            constexpr int NV = DT * 2;
            h8 va[4];
            auto ld_va = [&](int n) {
                const int t = n / 2, ks = n % 2;
                const int ch = 8 * ((2 * t + (l16 % 4) / 2) ^ sv);
                const h4 v0 = ld_tr(vbase + (32 * ks) * D + ch);
                const h4 v1 = ld_tr(vbase + (32 * ks + 16) * D + ch);
                return h8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            };
#pragma unroll
            for (int i = 0; i < LA; ++i)
                va[i] = ld_va(i);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0); // as for K
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int t = i / 2, ks = i % 2;
                if (i + LA < NV)
                    va[(i + LA) % 4] = ld_va(i + LA);
#pragma unroll
                for (int qt = 0; qt < QT; ++qt)
                    o[t][qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[i % 4], pb[ks][qt], o[t][qt], 0, 0, 0);
                if (i + LA < NV) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, QT, 0);
                }
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); // the next tile has landed in LDS
        __syncthreads();
    }

    // The cache planes of this workgroup's own positions: its diagonal tiles (j_diag
    // and, unless the prompt ends first, j_diag + 1) are the loop's last two, still in
    // the two tile buffers.  Quantised here, after the loop, so that the loop's waits
    // for the next tile never wait on these stores as well.
    for (int j = j_diag; j < n_tiles; ++j) {
        const _Float16 *lk = lds + (j & 1) * (Sh::LDS_K + Sh::LDS_V);
        quantise_tile<D, Meta>(g, pair, j, lk, lk + Sh::LDS_K);
    }
    __syncthreads(); // the tile buffers are read before the output rows reuse them

    // O = O^T / l.  Lane holds d = 16t + 4*g4 .. +3 of query 16*qt + l16; the wave's
    // rows are gathered in LDS (row pitch D + 8 halves) and written to HBM as whole
    // rows, 16 bytes per lane.
    constexpr int OP = D + 8;
    _Float16 *lo = lds + wave * Sh::QW * OP;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        float lt = l[qt];
        lt = xor_lanes16<true>(lt);
        lt = xor_lanes32<true>(lt);
        const float inv = 1.0f / lt;
#pragma unroll
        for (int t = 0; t < DT; ++t)
            *reinterpret_cast<h4 *>(lo + (16 * qt + l16) * OP + 16 * t + 4 * g4) =
                h4{(_Float16)(o[t][qt][0] * inv), (_Float16)(o[t][qt][1] * inv), (_Float16)(o[t][qt][2] * inv),
                   (_Float16)(o[t][qt][3] * inv)};
    }
    constexpr int LPR = D / 8;          // lanes per row
#pragma unroll
    for (int i = 0; i < Sh::QW * LPR / 64; ++i) {
        const int r = (64 * i + lane) / LPR, cc = (64 * i + lane) % LPR;
        const int qtok = qw0 + r;
        const uint4 x = *reinterpret_cast<const uint4 *>(lo + r * OP + 8 * cc);
        if (qtok < g.s_len)
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4b, x),
                                        reinterpret_cast<u32x4b *>(g.out + (((int64_t)bi * g.s_len + qtok) * g.a + ai) * D) + cc);
    }
}

// ===========================================================================
// head_dim 128: one (batch row, head) at a time per workgroup, persistent.
//
// A workgroup of 16 waves walks its (batch row, head) pairs one after the
// other; each pair's prompt is taken in passes of 256 queries (16 per wave),
// pass c seeing keys 0 .. 256c + 255.  The K/V tiles (64 keys) of the whole
// sequence of (pair, pass, tile) steps stream through a ring of three LDS
// stages, two tiles ahead of the one in use, across pass and pair
// boundaries, so the matrix cores never wait for a pass to start.  With four
// waves per SIMD, the softmax of one wave runs beside the products of
// another.  Pass c quantises its own positions' tiles (keys 256c ..
// 256c + 255) while they are in LDS, one K row chunk and one V row chunk per
// thread, so every prompt row is quantised exactly once.  The query rows of
// the next pass are fetched into registers two steps early, in the same
// order as the tiles, so the wait for a tile also covers them.
// ===========================================================================
namespace pp {
constexpr int D = 128;
constexpr int NW = 16;              // waves per workgroup
constexpr int NT = 64 * NW;         // threads
constexpr int QW = 16;              // queries per wave (one 16-row matrix-core tile)
constexpr int QP = QW * NW;         // queries per pass
constexpr int NSTG = 3;             // ring stages
constexpr int TILE_H = kKeys * D;   // halves per K or V tile (16 KB)
constexpr int STAGE_H = 2 * TILE_H; // K tile, then V tile
constexpr int KS = D / 32;          // k-steps of q.k
constexpr int DT = D / 16;          // 16-row tiles of O^T
} // namespace pp

struct PPArgs {
    const uint16_t *q, *k, *v; // fp16 [b][s_len][a][128]
    uint16_t *out;             // fp16 [b][s_len][a][128]
    uint32_t *k_codes, *v_codes;
    void *k_min, *k_scale, *v_min, *v_scale;
    int a, S, s_len;
    int pairs;     // b * a
    int passes;    // ceil(s_len / 256)
    int row_bytes; // a * 128 * 2: one token row of all heads
    int valid_bytes; // (s_len - 1) * row_bytes + 256: a head's prompt, from its token 0
    float c2, slack;
};

// The sequence of steps of one workgroup: pairs blockIdx.x, + gridDim.x, ...;
// passes 0 .. passes-1 of each; key tiles 0 .. nj-1 of each pass.  Uniform
// across the workgroup (scalar registers).  pair < 0: past the last step.
struct Step {
    int pair, c, j, nj;
    int64_t base; // byte offset of token 0 of the pair's head in q, k, v and out
};
__device__ __forceinline__ int pass_tiles(const PPArgs &g, int c)
{
    return (min(g.s_len, pp::QP * (c + 1)) + kKeys - 1) / kKeys;
}
__device__ __forceinline__ int64_t head_base(const PPArgs &g, int pair)
{
    const int bi = pair / g.a, ai = pair - bi * g.a;
    return ((int64_t)bi * g.s_len * g.a + ai) * pp::D * 2;
}
__device__ __forceinline__ Step first_step(const PPArgs &g)
{
    const int p = (int)blockIdx.x;
    return Step{p < g.pairs ? p : -1, 0, 0, pass_tiles(g, 0), p < g.pairs ? head_base(g, p) : 0};
}
__device__ __forceinline__ void next_step(const PPArgs &g, Step &u)
{
    if (u.pair < 0)
        return;
    if (++u.j < u.nj)
        return;
    u.j = 0;
    if (++u.c < g.passes) {
        u.nj = pass_tiles(g, u.c);
        return;
    }
    u.c = 0;
    u.pair += (int)gridDim.x;
    if (u.pair >= g.pairs) {
        u.pair = -1;
        return;
    }
    u.nj = pass_tiles(g, 0);
    u.base = head_base(g, u.pair);
}

// 16 bytes per lane, HBM -> LDS, as dma16, written out: the compiler does not
// see an LDS write here, so it adds no wait for these loads before LDS reads of
// other stages (it cannot tell the stages apart); the kernel's own waits and
// barriers order every tile.  r: the 128-bit buffer resource words.
typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4s rsrc_words(const void *p, int bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    return u32x4s{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu)),
                  (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}
__device__ __forceinline__ void dma16_raw(u32x4s r, _Float16 *dst, int voff)
{
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)dst);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m), "v"(voff), "s"(r)
                 : "memory", "m0");
}

// s_waitcnt encodings (gfx9): vmcnt in bits 3:0, expcnt 6:4, lgkmcnt 11:8.
// Through the builtin, so that the compiler's own wait insertion knows of them.
constexpr int kWaitVm2Lgkm0 = 0x0072; // vmcnt(2) lgkmcnt(0)
constexpr int kWaitVm0 = 0x0F70;      // vmcnt(0)

template <typename Meta>
__global__ __launch_bounds__(pp::NT, 1) void k_prefill_pp(PPArgs g)
{
    using namespace pp;
    using Sh = Shape<D>;
    // Three stages as three arrays, and the loop unrolled by three so that every
    // access names its stage: the compiler can then tell that reads of one stage
    // do not wait for the tile loads into the others.
    __shared__ __attribute__((aligned(16))) _Float16 lds0[STAGE_H];
    __shared__ __attribute__((aligned(16))) _Float16 lds1[STAGE_H];
    __shared__ __attribute__((aligned(16))) _Float16 lds2[STAGE_H];
    // Each wave's query rows of the current pass (16 rows, chunks swizzled as K's),
    // loaded by the wave itself and read only by it.
    __shared__ __attribute__((aligned(16))) _Float16 ldsq[NW * QW * D];
    auto stage = [&](auto K) -> _Float16 * {
        if constexpr (decltype(K)::value == 0)
            return lds0;
        else if constexpr (decltype(K)::value == 1)
            return lds1;
        else
            return lds2;
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;

    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64); // uniform: scalar registers
    const int l16 = lane % 16, g4 = lane / 16;
    const int tbytes = kKeys * g.row_bytes; // one key tile of a head

    // This thread's 16-byte piece of each tile: LDS position tid (row tid/16,
    // swizzled chunk tid%16), the unswizzled source chunk of K and of V.
    const int dr = tid / 16, dcs = tid % 16;
    const int dk = dr * g.row_bytes + 16 * (dcs ^ Sh::swz_k(dr));
    const int dv = dr * g.row_bytes + 16 * (dcs ^ Sh::swz_v(dr));
    auto issue = [&](const Step &u, _Float16 *st) {
        const int step = u.j * tbytes;
        const int nb = u.pair < 0 ? 0 : g.valid_bytes; // past the last step: zeros
        dma16_raw(rsrc_words(reinterpret_cast<const char *>(g.k) + u.base, nb), st + 512 * wave, dk + step);
        dma16_raw(rsrc_words(reinterpret_cast<const char *>(g.v) + u.base, nb), st + TILE_H + 512 * wave, dv + step);
    };
    // The wave's 16 query rows of pass u.c of pair u.pair, HBM -> its LDS rows:
    // piece 64i + lane is row (64i + lane)/16, swizzled chunk (64i + lane)%16.
    // Rows at or past the prompt's end read zeros (clamped to keep offsets small).
    _Float16 *const myq = ldsq + wave * QW * D;
    auto issue_q = [&](const Step &u) {
        const u32x4s r = rsrc_words(reinterpret_cast<const char *>(g.q) + u.base, u.pair < 0 ? 0 : g.valid_bytes);
#pragma unroll
        for (int i = 0; i < QW * D / 8 / 64; ++i) {
            const int pos = 64 * i + lane, qr = pos / 16, cs = pos % 16;
            const int off = min(u.c * QP + wave * QW + qr, g.s_len) * g.row_bytes + 16 * (cs ^ Sh::swz_k(qr));
            dma16_raw(r, myq + 512 * i, off);
        }
    };
    // The pass after the one of step u.
    auto next_pass = [&](Step u) {
        u.j = 0;
        if (++u.c < g.passes)
            return u;
        u.c = 0;
        u.pair += (int)gridDim.x;
        if (u.pair >= g.pairs)
            u.pair = -1;
        else
            u.base = head_base(g, u.pair);
        return u;
    };

    Step cu = first_step(g);
    if (cu.pair < 0)
        return;
    Step cd = cu;
    h8 qb[KS];
    issue_q(cu);
    issue(cd, lds0);
    next_step(g, cd);
    issue(cd, lds1);
    next_step(g, cd);

    f4 o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
        o[t] = f4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    // The output rows of a finished pass go out at the top of the next step,
    // before that step's loads, so that waiting for a tile never waits for them.
    bool out_due = false;
    int64_t out_base = 0;
    int out_q0 = 0;
    auto write_out = [&]() {
        if (out_q0 < g.s_len) {
            float lt = l;
            lt = xor_lanes16<true>(lt);
            lt = xor_lanes32<true>(lt);
            const float inv = __builtin_amdgcn_rcpf(lt);
            int ln = lane; // formed here rather than held across the loop
            asm volatile("" : "+v"(ln));
            const int qtok = out_q0 + ln % 16;
            if (qtok < g.s_len) {
                char *ob = reinterpret_cast<char *>(g.out) + out_base; // uniform
                const uint32_t off = (uint32_t)(qtok * g.row_bytes + 8 * (ln / 16));
#pragma unroll
                for (int t = 0; t < DT; ++t)
                    *reinterpret_cast<h4 *>(ob + off + 32 * t) =
                        h4{(_Float16)(o[t][0] * inv), (_Float16)(o[t][1] * inv), (_Float16)(o[t][2] * inv),
                           (_Float16)(o[t][3] * inv)};
            }
        }
#pragma unroll
        for (int t = 0; t < DT; ++t)
            o[t] = f4{0.f, 0.f, 0.f, 0.f};
        m = -INFINITY;
        l = 0.f;
    };

    // The V pieces quantised at the end of a step, stored at the top of the next
    // one (before its tile loads, like the output rows).
    QPiece vq{0u, 0u, 0.f, 0.f};
    bool vq_due = false;
    int64_t vq_slot0 = 0;
    int vq_tok0 = 0;
    auto put_vq = [&]() {
        int t = tid - 64 * (NW / 2);
        asm volatile("" : "+v"(t));
        const int tok = vq_tok0 + t / 8;
        if (tok < g.s_len)
            put_piece<Meta>(g.v_codes + vq_slot0 * (D / 8), static_cast<Meta *>(g.v_min) + vq_slot0 * (D / 64),
                            static_cast<Meta *>(g.v_scale) + vq_slot0 * (D / 64), tok, t % 8, vq);
    };
    // One step: the tile in stage RS, the loads two steps ahead into stage (RS+2)%3.
    auto run_step = [&](auto RS) -> bool {
        if (cu.pair < 0)
            return false;
        constexpr int rs = decltype(RS)::value;
        // This step's tile has landed in every thread (only the loads issued one
        // step ago may still be in flight: the issue order below keeps the stores
        // ahead of them), and every wave is done with the stage reused below.
        __builtin_amdgcn_s_waitcnt(kWaitVm2Lgkm0);
        __builtin_amdgcn_s_barrier();
        if (out_due) {
            write_out();
            out_due = false;
        }
        if (vq_due) {
            put_vq();
            vq_due = false;
        }
        if (cu.j == 0) {
            // A new pass: its query rows (loaded ahead of this step's tile, so they
            // have landed) into the Q^T operand registers -- lane: query l16,
            // d = 32kd + 8*g4 .. +7 -- then the next pass's rows into the same LDS
            // rows, once these reads are done.
            const int sq = Sh::swz_k(l16);
#pragma unroll
            for (int kd = 0; kd < KS; ++kd)
                qb[kd] = *reinterpret_cast<const h8 *>(myq + l16 * D + 8 * ((4 * kd + g4) ^ sq));
            __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
            issue_q(next_pass(cu));
        }
        const _Float16 *lk = stage(RS);
        const _Float16 *lv = lk + TILE_H;
        // This pass's own positions (keys 256c ..) are quantised while their tile
        // is in LDS, one 16-element piece of a row per thread: the K rows by
        // waves 0..7 here, the V rows by waves 8..15 after their products (stored
        // at the top of the next step), so that half of the waves run the codec
        // while the other half run the matrix cores.
        // own tile jj of the pass (keys 256c + 64jj ..): waves w < 4jj have no
        // query at or after its keys, so from jj = 1 on the low waves 0..7 take
        // the V rows too, before the others' products; on jj = 0 every wave has
        // products and the V rows go to waves 8..15 after theirs.
        const int jj = cu.j - cu.c * (QP / kKeys);
        const bool own = jj >= 0;
        if (own && wave < NW / 2) {
            int t = tid; // formed here rather than held across the loop
            asm volatile("" : "+v"(t));
            const int qr = t / 8, cc = t % 8;
            const int tok = cu.j * kKeys + qr;
            const int64_t slot0 = (int64_t)cu.pair * g.S; // plane bases of the pair (uniform)
            {
                const int sk = Sh::swz_k(qr);
                const uint4 x0 = *reinterpret_cast<const uint4 *>(lk + qr * D + 8 * ((2 * cc) ^ sk));
                const uint4 x1 = *reinterpret_cast<const uint4 *>(lk + qr * D + 8 * ((2 * cc + 1) ^ sk));
                QPiece qp;
                quant_lane16<Meta>(x0, x1, qp.w0, qp.w1, qp.mn, qp.sc); // every lane of the wave takes part (DPP)
                if (tok < g.s_len)
                    put_piece<Meta>(g.k_codes + slot0 * (D / 8), static_cast<Meta *>(g.k_min) + slot0 * (D / 64),
                                    static_cast<Meta *>(g.k_scale) + slot0 * (D / 64), tok, cc, qp);
            }
            if (jj > 0) {
                const int sv = Sh::swz_v(qr);
                const uint4 x0 = *reinterpret_cast<const uint4 *>(lv + qr * D + 8 * ((2 * cc) ^ sv));
                const uint4 x1 = *reinterpret_cast<const uint4 *>(lv + qr * D + 8 * ((2 * cc + 1) ^ sv));
                QPiece qp;
                quant_lane16<Meta>(x0, x1, qp.w0, qp.w1, qp.mn, qp.sc);
                if (tok < g.s_len)
                    put_piece<Meta>(g.v_codes + slot0 * (D / 8), static_cast<Meta *>(g.v_min) + slot0 * (D / 64),
                                    static_cast<Meta *>(g.v_scale) + slot0 * (D / 64), tok, cc, qp);
            }
        }
        // Two steps ahead: its tiles, into the stage released by the barrier above.
        __builtin_amdgcn_sched_barrier(0);
        issue(cd, stage(std::integral_constant<int, (rs + 2) % NSTG>{}));
        __builtin_amdgcn_sched_barrier(0);

        const int qw0 = cu.c * QP + wave * QW; // first query of this wave
        const int key0 = cu.j * kKeys;
        if (qw0 < g.s_len && key0 <= qw0 + QW - 1) {
            // S^T = K Q^T: st[c] holds keys 16c + 4*g4 + r, query l16.
            f4 st[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
                st[c] = f4{0.f, 0.f, 0.f, 0.f};
            constexpr int NSS = KS * 4, LA = 2;
            const int sk = Sh::swz_k(l16);
            auto ld_ka = [&](int n) {
                return *reinterpret_cast<const h8 *>(lk + (16 * (n % 4) + l16) * D + 8 * ((4 * (n / 4) + g4) ^ sk));
            };
            h8 ka[4];
#pragma unroll
            for (int i = 0; i < LA; ++i)
                ka[i] = ld_ka(i);
            // The first LA reads form a group of their own, ahead of the (read,
            // product) pairs: without it the scheduler fills the pairs' read slots
            // with them and every product waits on the read issued just before it.
            __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
            for (int i = 0; i < NSS; ++i) {
                if (i + LA < NSS)
                    ka[(i + LA) % 4] = ld_ka(i + LA);
                st[i % 4] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[i % 4], qb[i / 4], st[i % 4], 0, 0, 0);
                if (i + LA < NSS) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
            }
            if (key0 + kKeys - 1 > qw0) { // the diagonal tile: keys after the query are masked
                int ln = lane;
                asm volatile("" : "+v"(ln));
                const int rel = qw0 + ln % 16 - key0 - 4 * (ln / 16);
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (16 * c + r > rel)
                            st[c][r] = -INFINITY;
            }
            float mx = st[0][0];
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    mx = fmaxf(mx, st[c][r]);
            mx = xor_lanes16<false>(mx);
            mx = xor_lanes32<false>(mx);
            // The reference m moves only when some query's max exceeds it by more than
            // 8 (log2 units), as in k_prefill.
            if (__any(mx > m + g.slack)) {
                const float m_new = fmaxf(m, mx);
                const float alpha = exp2_fast((m - m_new) * g.c2);
                m = m_new;
                l *= alpha;
#pragma unroll
                for (int t = 0; t < DT; ++t)
                    o[t] *= alpha;
            }
            h8 pb[2];
            {
                const float mb = -m * g.c2;
                float ls = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float p = exp2_fast(__builtin_fmaf(st[c][r], g.c2, mb));
                        st[c][r] = p;
                        ls += p;
                    }
                l += ls;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pb[ks][r] = (_Float16)st[2 * ks][r];
                        pb[ks][4 + r] = (_Float16)st[2 * ks + 1][r];
                    }
            }
            // O^T += V^T P^T (operands as in k_prefill).  The read addresses are
            // formed here, not kept across the loop in 26 registers.
            const int vrow = 4 * g4 + l16 / 4;
            int sv = Sh::swz_v(vrow);
            asm volatile("" : "+v"(sv));
            const _Float16 *vbase = lv + vrow * D + 4 * (l16 % 2);
            constexpr int NV = DT * 2;
            h8 va[4];
            auto ld_va = [&](int n) {
                const int t = n / 2, ks = n % 2;
                const int ch = 8 * ((2 * t + (l16 % 4) / 2) ^ sv);
                const h4 v0 = ld_tr(vbase + (32 * ks) * D + ch);
                const h4 v1 = ld_tr(vbase + (32 * ks + 16) * D + ch);
                return h8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            };
#pragma unroll
            for (int i = 0; i < LA; ++i)
                va[i] = ld_va(i);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0); // as for K
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                if (i + LA < NV)
                    va[(i + LA) % 4] = ld_va(i + LA);
                o[i / 2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[i % 4], pb[i % 2], o[i / 2], 0, 0, 0);
                if (i + LA < NV) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
            }
        }
        if (jj == 0 && wave >= NW / 2) {
            int t = tid - 64 * (NW / 2);
            asm volatile("" : "+v"(t));
            const int qr = t / 8, cc = t % 8, sv = Sh::swz_v(qr);
            const uint4 x0 = *reinterpret_cast<const uint4 *>(lv + qr * D + 8 * ((2 * cc) ^ sv));
            const uint4 x1 = *reinterpret_cast<const uint4 *>(lv + qr * D + 8 * ((2 * cc + 1) ^ sv));
            quant_lane16<Meta>(x0, x1, vq.w0, vq.w1, vq.mn, vq.sc);
            vq_due = true;
            vq_slot0 = (int64_t)cu.pair * g.S;
            vq_tok0 = cu.j * kKeys;
        }
        if (cu.j + 1 == cu.nj) { // the pass ends: its output rows go out next step
            out_due = true;
            out_base = cu.base;
            out_q0 = qw0;
        }
        next_step(g, cu);
        next_step(g, cd);
        return true;
    };

    for (;;) {
        if (!run_step(S0{}) || !run_step(S1{}) || !run_step(S2{}))
            break;
    }
    if (out_due)
        write_out();
    if (vq_due)
        put_vq();
    // no tile load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
}

template <typename Meta>
int launch_prefill_pp(const CachePlanes &c, int b, const void *q, const void *k, const void *v, int s_len,
                      void *out, hipStream_t st)
{
    PPArgs g;
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
    g.pairs = b * c.a;
    g.passes = (s_len + pp::QP - 1) / pp::QP;
    g.row_bytes = c.a * pp::D * 2;
    // every offset formed (up to a key tile past the last prompt row) below 2^31
    if (((int64_t)s_len + 2 * kKeys) * g.row_bytes > 0x7FFFFFFF)
        return (int)hipErrorNotSupported;
    g.valid_bytes = (s_len - 1) * g.row_bytes + pp::D * 2;
    g.c2 = kLog2e / sqrtf((float)pp::D);
    g.slack = 8.0f / g.c2;
    const int grid = std::min(g.pairs, kPrefillCUs);
    hipLaunchKernelGGL((k_prefill_pp<Meta>), dim3((unsigned)grid), dim3(pp::NT), 0, st, g);
    return (int)hipGetLastError();
}

template <int D, typename Meta>
int launch_prefill_d(const CachePlanes &c, int b, const void *q, const void *k, const void *v, int s_len, void *out,
                     hipStream_t st)
{
    using Sh = Shape<D>;
    // Batch rows per launch: every byte offset the kernel forms (up to a tile and
    // a query tile past the last prompt row) stays below 2^31.
    const int64_t row_bytes = (int64_t)c.a * D * 2;
    const int64_t seq_bytes = (int64_t)s_len * row_bytes;
    const int64_t room = 0x7FFFFFFF - 2 * (int64_t)kKeys * row_bytes;
    if (seq_bytes > room)
        return (int)hipErrorNotSupported;
    const int b_step = (int)std::min<int64_t>(b, room / seq_bytes);
    PrefillArgs g;
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
    g.c2 = kLog2e / sqrtf((float)D);
    g.slack = 8.0f / g.c2;
    for (int b0 = 0; b0 < b; b0 += b_step) {
        const int bc = std::min(b_step, b - b0);
        const int64_t elem0 = (int64_t)b0 * s_len * c.a * D;
        g.q = static_cast<const uint16_t *>(q) + elem0;
        g.k = static_cast<const uint16_t *>(k) + elem0;
        g.v = static_cast<const uint16_t *>(v) + elem0;
        g.out = static_cast<uint16_t *>(out) + elem0;
        g.pair0 = (int64_t)b0 * c.a;
        g.bytes = (int)(bc * seq_bytes);
        g.total = (int64_t)bc * c.a * g.n_qtiles;
        g.chunk = (g.total + 7) / 8;
        const int64_t grid = 8 * g.chunk;
        if (grid > 0x7FFFFFFF)
            return (int)hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((k_prefill<D, Meta>), dim3((unsigned)grid), dim3(kThreads), 0, st, g);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return (int)e;
    }
    return 0;
}

template <typename Meta>
int launch_prefill_m(const CachePlanes &c, int b, const void *q, const void *k, const void *v, int s_len, void *out,
                     hipStream_t st)
{
    switch (c.d) {
    case 64: return launch_prefill_d<64, Meta>(c, b, q, k, v, s_len, out, st);
    case 128: return launch_prefill_pp<Meta>(c, b, q, k, v, s_len, out, st);
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
