// HIP kernels for gfx950: int4 group-wise KV-cache quantisation, dense
// decode attention over the int4 cache (with a split-context reduce pass),
// and top-k sparse decode attention.
//
// Definitions followed (page titles and sections):
//  * codec: "FlexGen研究学术报告" section 三.2(C) -- group-wise asymmetric
//    4-bit quantisation, 64 contiguous elements per group, dequantised to
//    FP16 before compute; group axis = head_dim, min/max affine code with
//    scale (max-min)/15 and round-half-even codes (readings stated in
//    include/kvq4.h);
//  * decode attention: the FlexGen blog, section "解码阶段":
//    t_out = softmax(t_Q x_K^T / sqrt(.)) x_V, stopping before W_O, with the
//    per-head 1/sqrt(d_k) scale of eq. (2) in the efficient-inference survey
//    notes;
//  * sparse variant: the report's section 三.2(C), top-10% sparse attention.
//
// Everything here streams HBM once: the path is bandwidth-bound (the survey
// notes' "Efficiency Analysis" gives decoding a very low compute-to-memory
// ratio), so the kernels are shaped around 16-byte coalesced loads, no LDS
// staging of the cache, and a VALU budget of a few operations per element.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "kvq4.h"
#include "kvq4_device.h"
#include "kvq4_launch.h"

// The workspace of decode_attention_q4_noalloc: the split partials (max, sum
// and unnormalised output per split and (batch row, head)) live in this
// library-owned device array instead of a caller buffer.  Each GPU the
// library runs on holds its own copy (KVQ_NOALLOC_SCRATCH_BYTES) until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device address: host code uses only the per-device address that
// noalloc_scratch() obtains from the runtime.
static __device__ __align__(256) float scratch[KVQ_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace kvq {
namespace {

// A min or scale of either metadata type (binary32 or binary16), widened to
// binary32 (exact).
__device__ __forceinline__ float ld_meta(const float *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float ld_meta(const _Float16 *p) { return (float)__builtin_nontemporal_load(p); }

// ---------------------------------------------------------------------------
// Nibble unpack.  A 32-bit word of codes holds elements e0..e7 (nibble k at
// bits 4k..4k+3, even element in the low nibble of each byte).  Each 16-bit
// half holds two codes in its low byte (bits 0..3 and 4..7); one shift by 8
// brings the two codes of its high byte down.  Masking then gives the pairs
// (e0,e4), (e1,e5) from the word and (e2,e6), (e3,e7) from the shifted word,
// one instruction each, in two forms:
//  * keys, for v_dot2_f32_f16 (which flushes binary16 subnormals): OR-ing the
//    binary16 pattern of 1024 onto a nibble at bits 0..3 gives exactly
//    1024 + c (the fraction's bit 0 weighs 1 at exponent 10), and one packed
//    binary16 subtraction of 1024 leaves c itself (exact); OR-ing 64 onto a
//    nibble at bits 4..7 gives 64 + c (bit 4 weighs 1 at exponent 6), kept
//    biased.  The dot's binary32 partial sums then stay near 64 * sum q_odd
//    + sum q_i c_i: keeping 1024 + c for the even elements made them about
//    1024 * sum q_even, and with queries and keys of outlier channels (x8)
//    their rounding alone moved a score by ~1e-3.
//  * values, for the mixed-precision FMA (which keeps binary16 subnormals):
//    the masked halves alone are the subnormals c * 2^-24 (bits 0..3) and
//    c * 2^-20 (bits 4..7), with no bias to remove.
// ---------------------------------------------------------------------------
constexpr uint32_t kLoNib = 0x000F000Fu;
constexpr uint32_t kHiNib = 0x00F000F0u;
constexpr float kBiasHi = 64.0f;   // keys: bias of e1, e3, e5, e7 (e0, e2, e4, e6 carry none)
constexpr float kTwo24 = 16777216.0f;

// The OR constants are held in VGPRs (opaque to the compiler) so each key pair
// compiles to a single v_and_or_b32 with the mask in an SGPR: GFX9's VOP3
// takes no literal and at most one scalar operand.
struct Magic {
    uint32_t lo, hi;
};
__device__ __forceinline__ Magic magic_vgprs()
{
    Magic m;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m.lo));
    asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(m.hi));
    return m;
}

__device__ __forceinline__ float fdot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

// One lane's 32-element slice of q, regrouped into the unpack's pair order,
// plus its sum (for the group min) and the key bias sum_i q_i * bias_i
// (64 * the sum of the odd elements).
// v_dot2_f32_f16 flushes binary16 subnormals, so a subnormal query element
// (|q_i| < 2^-14) is taken as 0 in all three: the score then misses only
// q_i * k_i for those elements (at most 2^-14 |k_i| each), instead of the
// bias term q_i * (bias_i + c_i) * scale a flushed dot against an unflushed
// bias sum would leave in every score.
struct QSlice {
    uint32_t qp[16];
    float qsum;
    float qbias;
};

// The lane's 32 query elements as loaded (4 x 16 bytes).
struct QRaw {
    uint4 v[4];
};

__device__ __forceinline__ QRaw load_q_raw(const uint4 *__restrict__ qrow)
{
    QRaw r;
#pragma unroll
    for (int w = 0; w < 4; ++w)
        r.v[w] = qrow[w];
    return r;
}

// The two binary16 values of a word with every subnormal (exponent field 0)
// replaced by +0.
__device__ __forceinline__ uint32_t flush_f16_subnormals(uint32_t w)
{
    const uint32_t keep_lo = (w & 0x00007C00u) ? 0x0000FFFFu : 0u;
    const uint32_t keep_hi = (w & 0x7C000000u) ? 0xFFFF0000u : 0u;
    return w & (keep_lo | keep_hi);
}

__device__ __forceinline__ QSlice q_slice(const QRaw &r)
{
    QSlice s;
    float even = 0.0f, odd = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        // elements 8w..8w+7: x=(e0,e1) y=(e2,e3) z=(e4,e5) w=(e6,e7)
        const uint4 v = make_uint4(flush_f16_subnormals(r.v[w].x), flush_f16_subnormals(r.v[w].y),
                                   flush_f16_subnormals(r.v[w].z), flush_f16_subnormals(r.v[w].w));
        s.qp[4 * w + 0] = (v.x & 0xFFFFu) | (v.z << 16);
        s.qp[4 * w + 1] = (v.x >> 16) | (v.z & 0xFFFF0000u);
        s.qp[4 * w + 2] = (v.y & 0xFFFFu) | (v.w << 16);
        s.qp[4 * w + 3] = (v.y >> 16) | (v.w & 0xFFFF0000u);
        even += h2f_lo(v.x) + h2f_lo(v.y) + h2f_lo(v.z) + h2f_lo(v.w);
        odd += h2f_hi(v.x) + h2f_hi(v.y) + h2f_hi(v.z) + h2f_hi(v.w);
    }
    s.qsum = even + odd;
    s.qbias = kBiasHi * odd;
    return s;
}

// (1024 + c0, 1024 + c1) -> (c0, c1), exact, one packed binary16 subtraction.
__device__ __forceinline__ uint32_t unbias1024(uint32_t k)
{
    const f16x2 m = {(_Float16)1024.0f, (_Float16)1024.0f};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, k) - m);
}

// sum_i q_i * c_i over the lane's 32 elements: the dot against the key form
// (c for the even elements, 64 + c for the odd ones) started at -qbias.
__device__ __forceinline__ float dot_keys(const QSlice &q, const uint4 kx, const Magic mg)
{
    const uint32_t w[4] = {kx.x, kx.y, kx.z, kx.w};
    float acc = -q.qbias;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t y = w[j] >> 8;
        acc = fdot2(q.qp[4 * j + 0], unbias1024((w[j] & kLoNib) | mg.lo), acc);
        acc = fdot2(q.qp[4 * j + 1], (w[j] & kHiNib) | mg.hi, acc);
        acc = fdot2(q.qp[4 * j + 2], unbias1024((y & kLoNib) | mg.lo), acc);
        acc = fdot2(q.qp[4 * j + 3], (y & kHiNib) | mg.hi, acc);
    }
    return acc;
}

// acc[i] += ps * c_i for the lane's 32 elements (natural order), value form;
// ps_lo = ps * 2^24.
__device__ __forceinline__ void axpy_values(float (&acc)[32], float ps_lo, const uint4 vx)
{
    const float ps_hi = ps_lo * 0.0625f;
    const uint32_t w[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t y = w[j] >> 8;
        const uint32_t p0 = w[j] & kLoNib, p1 = w[j] & kHiNib, p2 = y & kLoNib, p3 = y & kHiNib;
        acc[8 * j + 0] = __builtin_fmaf(ps_lo, h2f_lo(p0), acc[8 * j + 0]);
        acc[8 * j + 4] = __builtin_fmaf(ps_lo, h2f_hi(p0), acc[8 * j + 4]);
        acc[8 * j + 1] = __builtin_fmaf(ps_hi, h2f_lo(p1), acc[8 * j + 1]);
        acc[8 * j + 5] = __builtin_fmaf(ps_hi, h2f_hi(p1), acc[8 * j + 5]);
        acc[8 * j + 2] = __builtin_fmaf(ps_lo, h2f_lo(p2), acc[8 * j + 2]);
        acc[8 * j + 6] = __builtin_fmaf(ps_lo, h2f_hi(p2), acc[8 * j + 6]);
        acc[8 * j + 3] = __builtin_fmaf(ps_hi, h2f_lo(p3), acc[8 * j + 3]);
        acc[8 * j + 7] = __builtin_fmaf(ps_hi, h2f_hi(p3), acc[8 * j + 7]);
    }
}

// Sum over the LPT lanes that hold one token row.
template <int LPT>
__device__ __forceinline__ float token_sum(float v)
{
    if constexpr (LPT >= 2)
        v += dpp<kQuadXor1>(v);
    if constexpr (LPT >= 4)
        v += dpp<kQuadXor2>(v);
    if constexpr (LPT >= 8)
        v += dpp<kHalfRowMirror>(v);
    return v;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ===========================================================================
// Quantise.  Each lane loads 8 fp16 values (16 bytes); 8 consecutive lanes
// hold one 64-element group and reduce its min/max with three DPP steps.
// R > 1 (a prompt): workgroup x = (pair, chunk of RPB*R tokens of that pair),
// so the pair and its (batch row, head) are uniform across the workgroup
// (scalar arithmetic) and lanes with consecutive rows write consecutive cache
// slots; the 16-byte reads are whole 256-byte rows.  R = 1 (one appended
// token per pair): RPB consecutive pairs per workgroup.
// ===========================================================================
// n / d for 32-bit n (Granlund & Montgomery, "Division by invariant integers
// using multiplication", the round-up multiplier): l = ceil(log2 d),
// mul = floor(2^32 (2^l - d) / d) + 1, q = (t + ((n - t) >> min(l,1))) >> max(l-1,0)
// with t = the high half of mul * n.
struct FastDiv {
    uint32_t mul, sh1, sh2;
};
__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f)
{
    const uint32_t t = __umulhi(n, f.mul);
    return (t + ((n - t) >> f.sh1)) >> f.sh2;
}
FastDiv make_fast_div(uint32_t d)
{
    int l = 0;
    while ((1ull << l) < d)
        ++l;
    const uint64_t mul = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{(uint32_t)mul, (uint32_t)std::min(l, 1), (uint32_t)std::max(l - 1, 0)};
}

template <int D, int R, typename Meta>
__global__ __launch_bounds__(256) void k_quantize(const uint4 *__restrict__ k_src, const uint4 *__restrict__ v_src,
                                                  int pairs, int s_src, int chunks, FastDiv by_chunks, int a,
                                                  FastDiv by_a, int S, int t_dst0,
                                                  uint32_t *__restrict__ k_codes, uint32_t *__restrict__ v_codes,
                                                  Meta *__restrict__ k_min, Meta *__restrict__ k_scale,
                                                  Meta *__restrict__ v_min, Meta *__restrict__ v_scale)
{
    constexpr int LPR = D / 8;   // lanes per token row
    constexpr int RPB = 256 / LPR;
    constexpr int G = D / 64;
    const bool is_v = blockIdx.y != 0;
    const uint4 *__restrict__ src = is_v ? v_src : k_src;
    uint32_t *__restrict__ codes = is_v ? v_codes : k_codes;
    Meta *__restrict__ mins = is_v ? v_min : k_min;
    Meta *__restrict__ scales = is_v ? v_scale : k_scale;
    const int lir = threadIdx.x % LPR;
    const int rib = threadIdx.x / LPR; // row within the workgroup's RPB

    int pair, t0;
    if constexpr (R == 1) {
        pair = min((int)blockIdx.x * RPB + rib, pairs - 1); // lanes past the last pair redo it, storing nothing
        t0 = 0;
    } else {
        pair = (int)fast_div(blockIdx.x, by_chunks);
        t0 = ((int)blockIdx.x - pair * chunks) * (RPB * R) + rib;
    }
    const int bi = (int)fast_div((uint32_t)pair, by_a);
    const int ai = pair - bi * a;
    const uint4 *__restrict__ row0 = src + ((int64_t)bi * s_src * a + ai) * LPR + lir; // token 0 of the pair
    const int64_t tok_stride = (int64_t)a * LPR;

    uint4 x[R];
    bool ok[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int t = t0 + u * RPB;
        ok[u] = R == 1 ? (int)blockIdx.x * RPB + rib < pairs : t < s_src;
        x[u] = ld_stream16(row0 + (int64_t)min(t, s_src - 1) * tok_stride);
    }
    const int64_t slot0 = (int64_t)pair * S + t_dst0 + t0;
#pragma unroll
    for (int u = 0; u < R; ++u) {
        uint32_t word;
        float mn, scale;
        quant_lane8<Meta>(x[u], word, mn, scale);
        // Nontemporal stores: cache rows are read back only by a later launch,
        // and ordinary stores left dirty lines whose write-back slowed the next
        // decode launch by ~5% (measured on MI355X).
        if (ok[u]) {
            const int64_t slot = slot0 + u * RPB;
            __builtin_nontemporal_store(word, codes + slot * (D / 8) + lir);
            if ((lir & 7) == 0) {
                __builtin_nontemporal_store((Meta)mn, mins + slot * G + (lir >> 3));
                __builtin_nontemporal_store((Meta)scale, scales + slot * G + (lir >> 3));
            }
        }
    }
}

// One iteration of the dense decode loop for one lane: UU tokens spaced TPW
// apart starting at token tb (tokens >= t_end are masked; their loads are
// clamped to t_end-1 so they stay inside the written cache).  Updates the
// lane's online-softmax state (m, l in log2 units; bsum collects the folded
// min terms; acc the biased P.V sums).
// One token row in the attention lane layout (see append_rows).
struct NewRow {
    uint4 kx, vx;
    float km, ks, vm, vs;
};

// The streams of one (batch row, head): plane bases that are uniform across
// the wave (scalar registers), and the lane's 32-bit offsets of its slice
// inside a token row.  Loads then take the scalar-base + 32-bit-offset
// address form instead of a per-lane 64-bit pointer (saves ~2 VALU per load).
template <typename Meta>
struct CacheRow {
    const uint8_t *__restrict__ kb;
    const uint8_t *__restrict__ vb;
    const Meta *__restrict__ kmb;
    const Meta *__restrict__ ksb;
    const Meta *__restrict__ vmb;
    const Meta *__restrict__ vsb;
    uint32_t code_off; // part * 16 bytes
    uint32_t meta_off; // sizeof(Meta) * group index g, bytes
};

// Element at a 32-bit byte offset from a wave-uniform base.
template <typename T>
__device__ __forceinline__ const T *at_byte(const T *base, uint32_t off)
{
    return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + off);
}

template <int D, typename Meta>
__device__ __forceinline__ CacheRow<Meta> cache_row(const uint8_t *kc, const uint8_t *vc, const Meta *kmin, const Meta *ksc,
                                                 const Meta *vmin, const Meta *vsc, int pair, int S, int part)
{
    constexpr int G = D / 64;
    const int64_t p = __builtin_amdgcn_readfirstlane(pair); // wave-uniform by construction
    const int64_t cb = p * S * (D / 2), mb = p * S * G;
    return {kc + cb, vc ? vc + cb : nullptr, kmin + mb, ksc + mb, vmin ? vmin + mb : nullptr,
            vsc ? vsc + mb : nullptr, (uint32_t)part * 16u, (uint32_t)(part >> 1) * (uint32_t)sizeof(Meta)};
}

// The cache rows of one iteration: UU token rows per lane (rows tb, tb + TPW,
// ...), each with its K and V code words and min/scale.  Rows at or past
// t_end load row t_end - 1 (in bounds) and are flagged invalid.
template <int UU>
struct KVRows {
    uint4 kx[UU], vx[UU];
    float km[UU], ks[UU], vm[UU], vs[UU];
    bool valid[UU];
};

// The K half (KV = false: K codes and min/scale, and the valid flags) or the
// V half (KV = true) of load_kv_rows.
template <int D, int UU, bool KV, typename Meta>
__device__ __forceinline__ void load_rows_half(const CacheRow<Meta> &cr, int tb, int t_end, KVRows<UU> &r)
{
    constexpr int LPT = D / 32;
    constexpr int TPW = 64 / LPT;
    constexpr int G = D / 64;
#pragma unroll
    for (int u = 0; u < UU; ++u) {
        const int t = tb + u * TPW;
        const bool valid = t < t_end;
        const uint32_t tcl = (uint32_t)(valid ? t : t_end - 1);
        const uint32_t co = tcl * (D / 2) + cr.code_off, mo = tcl * (uint32_t)(sizeof(Meta) * G) + cr.meta_off;
        if constexpr (!KV) {
            r.valid[u] = valid;
            r.kx[u] = ld_stream16(cr.kb + co);
            r.km[u] = ld_meta(at_byte(cr.kmb, mo));
            r.ks[u] = ld_meta(at_byte(cr.ksb, mo));
        } else {
            r.vx[u] = ld_stream16(cr.vb + co);
            r.vm[u] = ld_meta(at_byte(cr.vmb, mo));
            r.vs[u] = ld_meta(at_byte(cr.vsb, mo));
        }
    }
}

template <int D, int UU, typename Meta>
__device__ __forceinline__ void load_kv_rows(const CacheRow<Meta> &cr, int tb, int t_end, KVRows<UU> &r)
{
    constexpr int LPT = D / 32;
    constexpr int TPW = 64 / LPT;
    constexpr int G = D / 64;
#pragma unroll
    for (int u = 0; u < UU; ++u) {
        const int t = tb + u * TPW;
        r.valid[u] = t < t_end;
        const uint32_t tcl = (uint32_t)(r.valid[u] ? t : t_end - 1);
        const uint32_t co = tcl * (D / 2) + cr.code_off, mo = tcl * (uint32_t)(sizeof(Meta) * G) + cr.meta_off;
        r.kx[u] = ld_stream16(cr.kb + co);
        r.vx[u] = ld_stream16(cr.vb + co);
        r.km[u] = ld_meta(at_byte(cr.kmb, mo));
        r.ks[u] = ld_meta(at_byte(cr.ksb, mo));
        r.vm[u] = ld_meta(at_byte(cr.vmb, mo));
        r.vs[u] = ld_meta(at_byte(cr.vsb, mo));
    }
}

// Scores of the rows, online-softmax update of (m, l, bsum, acc).  m is a
// reference, not the running maximum: it moves, and l, bsum and acc are
// rescaled, only when a score exceeds it by more than kSlack (log2 units).
// The probabilities 2^(z - m) then stay below 2^kSlack, far from the binary32
// range at any context, and the rescale runs a few times per token sequence
// instead of at nearly every iteration (with 64 lanes, some lane's maximum
// moves almost every time).  The merges over lanes, waves and splits take any
// reference.
constexpr float kSlack = 8.0f;

template <int D, int UU>
__device__ __forceinline__ void attend_kv_rows(const KVRows<UU> &r, const QSlice &qs, const Magic mg, float c2,
                                               float &m, float &l, float &bsum, float (&acc)[32])
{
    constexpr int LPT = D / 32;
    float z[UU];
    float zmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < UU; ++u) {
        const float dq = dot_keys(qs, r.kx[u], mg);
        float sp = __builtin_fmaf(r.ks[u], dq, r.km[u] * qs.qsum);
        sp = token_sum<LPT>(sp);
        z[u] = r.valid[u] ? sp * c2 : -INFINITY;
        zmax = fmaxf(zmax, z[u]);
    }
    const bool grow = zmax > m + kSlack; // false while every score seen is -inf
    const float m_new = grow ? zmax : m;
    const float mref = (m_new == -INFINITY) ? 0.0f : m_new;
    if (__any(grow)) {
        const float alpha = exp2_fast(m - mref); // 1 where m stays, 0 from m = -inf
        l *= alpha;
        bsum *= alpha;
#pragma unroll
        for (int i = 0; i < 32; ++i)
            acc[i] *= alpha;
    }
    m = m_new;
#pragma unroll
    for (int u = 0; u < UU; ++u) {
        const float p = exp2_fast(z[u] - mref);
        l += p;
        bsum = __builtin_fmaf(p, r.vm[u], bsum);
        axpy_values(acc, p * (r.vs[u] * kTwo24), r.vx[u]);
    }
}

template <int D, int UU, bool NEWROW = false, typename Meta>
__device__ __forceinline__ void decode_iter(const CacheRow<Meta> &cr, int tb, int t_end, const QSlice &qs, const Magic mg,
                                            float c2, float &m, float &l, float &bsum, float (&acc)[32],
                                            const NewRow nr = NewRow{}, int t_new = -1)
{
    constexpr int TPW = 64 / (D / 32);
    KVRows<UU> r;
    load_kv_rows<D, UU>(cr, tb, t_end, r);
    if constexpr (NEWROW) {
#pragma unroll
        for (int u = 0; u < UU; ++u) {
            if (tb + u * TPW == t_new) {
                r.kx[u] = nr.kx;
                r.vx[u] = nr.vx;
                r.km[u] = nr.km;
                r.ks[u] = nr.ks;
                r.vm[u] = nr.vm;
                r.vs[u] = nr.vs;
            }
        }
    }
    attend_kv_rows<D, UU>(r, qs, mg, c2, m, l, bsum, acc);
}

// Fused append.  The wave whose range ends at the new slot quantises the new
// token's K and V rows of its (batch row, head) and stores them into slot
// `pos` for later steps.  It does not wait for or read back those stores:
// the row is also returned in the attention lane layout (lane `part` gets
// code words 4*part..4*part+3 and the min/scale of group part/2) and is
// substituted for slot `pos` in the wave's last iteration.  The values are
// the stored ones, so the result is identical to a separate append.
// The lane's 16 bytes of the new K row (lanes 0..D/8-1) or V row (lanes
// D/8..2D/8-1); lanes past 2*D/8 repeat the V row.  Loaded at the start of the
// tail wave so the load latency is hidden behind its main loop.
template <int D>
__device__ __forceinline__ uint4 load_new_row(const uint4 *__restrict__ k_new, const uint4 *__restrict__ v_new,
                                              int64_t pair, int lane)
{
    constexpr int LPR = D / 8;
    return ld_stream16((lane < LPR ? k_new : v_new) + pair * (D / 8) + lane % LPR);
}

template <int D, typename Meta>
__device__ __forceinline__ NewRow append_rows(const uint4 x, int64_t pair, int64_t pos, int S, uint8_t *kc,
                                              uint8_t *vc, Meta *kmin, Meta *ksc, Meta *vmin, Meta *vsc, int lane)
{
    constexpr int LPR = D / 8;
    constexpr int G = D / 64;
    constexpr int LPT = D / 32;
    const int which = min(lane / LPR, 1);
    const int lir = lane % LPR;
    uint32_t word;
    float mn, scale;
    quant_lane8<Meta>(x, word, mn, scale);
    if (lane < 2 * LPR) {
        const int64_t slot = pair * S + pos;
        __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(which ? vc : kc) + slot * (D / 8) + lir);
        if ((lir & 7) == 0) {
            __builtin_nontemporal_store((Meta)mn, (which ? vmin : kmin) + slot * G + (lir >> 3));
            __builtin_nontemporal_store((Meta)scale, (which ? vsc : ksc) + slot * G + (lir >> 3));
        }
    }
    const int part = lane % LPT, g = part >> 1;
    NewRow r;
    r.kx = make_uint4(__shfl(word, 4 * part), __shfl(word, 4 * part + 1), __shfl(word, 4 * part + 2),
                      __shfl(word, 4 * part + 3));
    r.vx = make_uint4(__shfl(word, LPR + 4 * part), __shfl(word, LPR + 4 * part + 1),
                      __shfl(word, LPR + 4 * part + 2), __shfl(word, LPR + 4 * part + 3));
    r.km = __shfl(mn, 8 * g);
    r.ks = __shfl(scale, 8 * g);
    r.vm = __shfl(mn, LPR + 8 * g);
    r.vs = __shfl(scale, LPR + 8 * g);
    return r;
}

// The value of v held by another lane: for OFF < 16 the lane OFF places
// earlier in the same 16-lane row (DPP row rotation, no LDS), else lane ^ OFF.
template <int OFF>
__device__ __forceinline__ float lane_peer(float v)
{
    if constexpr (OFF < 16)
        return dpp<0x120 + OFF>(v); // row_ror:OFF
    else
        return __shfl_xor(v, OFF);
}

// Online-softmax states (m, l, acc) merged over the lanes congruent modulo
// OFF0: at each step a lane merges its state with lane_peer's.  The merge
// (max, rescale, add) is associative and commutative, so after the steps
// OFF0, 2 OFF0, .. 32 every lane holds the merge of its whole class.
template <int OFF>
__device__ __forceinline__ void merge_token_lanes(float &m, float &l, float (&acc)[32])
{
    if constexpr (OFF < 64) {
        const float mo = lane_peer<OFF>(m);
        const float lo = lane_peer<OFF>(l);
        const float M = fmaxf(m, mo);
        const float Mr = (M == -INFINITY) ? 0.0f : M;
        const float a1 = exp2_fast(m - Mr), a2 = exp2_fast(mo - Mr);
        l = l * a1 + lo * a2;
#pragma unroll
        for (int i = 0; i < 32; ++i)
            acc[i] = acc[i] * a1 + lane_peer<OFF>(acc[i]) * a2;
        m = M;
        merge_token_lanes<OFF * 2>(m, l, acc);
    }
}

// ===========================================================================
// Dense decode attention.
//
// Lane layout: a token row of d codes is d/2 bytes = LPT lanes x 16 bytes, so
// one 16-byte load per lane covers TPW = 64/LPT tokens per wave (1 KB for
// d = 128).  Lane `part` = lane % LPT owns elements 32*part..32*part+31 of
// every token it visits (all inside group part/2); lane lt = lane / LPT walks
// its own token sequence with a private online-softmax state.  The states of
// the TPW token lanes are merged once at the end (log-sum-exp), then across
// the waves sharing a (batch row, head), then (split > 1) by k_reduce.
//
// The dequantisation x = min + c*scale is folded out of the inner loops:
//   q.x      = scale * sum q_i(64+c_i) + (min - 64*scale) * sum q_i
//   sum p.x  = sum (p*scale)(64+c_i)   + sum p*(min - 64*scale)
// so the per-element work is the nibble unpack plus one dot2 (K) or one
// mixed-precision FMA (V).  Scores are kept in log2 units (z = s*log2e/sqrt(d)).
// ===========================================================================
template <int D, int U, int WPP, typename Meta>
__global__ __launch_bounds__(256) void k_decode(uint8_t *kc, uint8_t *vc, Meta *kmin, Meta *ksc, Meta *vmin, Meta *vsc,
                                                const uint4 *__restrict__ q, uint4 *__restrict__ out,
                                                float *__restrict__ ws, int pairs, int S, int T, int splits,
                                                int split_len, float c2, const uint4 *__restrict__ k_new,
                                                const uint4 *__restrict__ v_new)
{
    constexpr int LPT = D / 32;
    constexpr int TPW = 64 / LPT;
    constexpr int PPB = 4 / WPP;
    constexpr int TPI = U * TPW;
    __shared__ float sm_acc[WPP > 1 ? 4 : 1][WPP > 1 ? D : 1];
    __shared__ float sm_ml[4][2];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wp = wave % WPP;
    const int pslot = wave / WPP;
    const int split = blockIdx.x % splits;
    const int pair = (blockIdx.x / splits) * PPB + pslot;
    const bool pair_ok = pair < pairs;
    const int64_t pc = pair_ok ? pair : pairs - 1;
    const int part = lane % LPT;
    const int lt = lane / LPT;
    // This split's tokens [t0, t1), cut into WPP contiguous per-wave ranges
    // (whole TPW-token rows so only the last wave has a ragged end).
    const int t0 = split * split_len;
    const int t1 = min(T, t0 + split_len);
    const int n_tok = max(0, t1 - t0);
    const int per_wave = ((n_tok + WPP - 1) / WPP + TPW - 1) / TPW * TPW;
    const int w_begin = min(t1, t0 + wp * per_wave);
    const int t_end = min(t1, w_begin + per_wave);
    const int n_full = (t_end - w_begin) / TPI;            // iterations with all U rows valid
    const int n_rest = (t_end - w_begin - n_full * TPI + TPW - 1) / TPW; // single-row tail iterations
    // Fused append (k_new != null): the wave whose range ends at the new slot
    // T-1 quantises and stores it, and uses the register copy in its last row.
    const bool tail_wave = k_new != nullptr && pair_ok && t_end == T && w_begin < t_end; // wave-uniform
    // The tail wave's rows: all but the last TPW-row chunk as usual, then that
    // chunk with the new row substituted for slot T-1.
    const int last = w_begin + (t_end - 1 - w_begin) / TPW * TPW;
    const int nf = tail_wave ? (last - w_begin) / TPI : n_full; // full iterations
    const CacheRow<Meta> cr = cache_row<D, Meta>(kc, vc, kmin, ksc, vmin, vsc, (int)pc, S, part);
    uint4 new_raw = make_uint4(0, 0, 0, 0);
    if (tail_wave)
        new_raw = load_new_row<D>(k_new, v_new, pc, lane);
    // The first iteration's K rows are requested right behind the query, so
    // the wave's first memory round trip carries both; its V rows follow the
    // query's processing and arrive during the scores.
    const QRaw qraw = load_q_raw(q + pc * (D / 8) + part * 4);
    int tb = w_begin + lt;
    KVRows<U> first;
    if (nf > 0)
        load_rows_half<D, U, false>(cr, tb, t_end, first);
    const QSlice qs = q_slice(qraw);
    const Magic mg = magic_vgprs();
    if (nf > 0)
        load_rows_half<D, U, true>(cr, tb, t_end, first);

    float m = -INFINITY, l = 0.0f, bsum = 0.0f;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i)
        acc[i] = 0.0f;

    if (nf > 0) {
        attend_kv_rows<D, U>(first, qs, mg, c2, m, l, bsum, acc);
        tb += TPI;
    }
    if (!tail_wave) {
        for (int it = 1; it < n_full; ++it, tb += TPI)
            decode_iter<D, U>(cr, tb, t_end, qs, mg, c2, m, l, bsum, acc);
        for (int it = 0; it < n_rest; ++it, tb += TPW)
            decode_iter<D, 1>(cr, tb, t_end, qs, mg, c2, m, l, bsum, acc);
    } else {
        // the new row is quantised and stored right after the first iteration
        // (its load arrived with the first rows), so the codec and its lane
        // exchanges overlap the rest of the wave's stream instead of ending it
        const NewRow nr = append_rows<D, Meta>(new_raw, pc, T - 1, S, kc, vc, kmin, ksc, vmin, vsc, lane);
        const int nr1 = (last - w_begin - nf * TPI) / TPW;
        for (int it = 1; it < nf; ++it, tb += TPI)
            decode_iter<D, U>(cr, tb, t_end, qs, mg, c2, m, l, bsum, acc);
        for (int it = 0; it < nr1; ++it, tb += TPW)
            decode_iter<D, 1>(cr, tb, t_end, qs, mg, c2, m, l, bsum, acc);
        decode_iter<D, 1, true>(cr, tb, t_end, qs, mg, c2, m, l, bsum, acc, nr, T - 1);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i)
        acc[i] += bsum;

    // Merge the TPW token lanes that share `part`.
    merge_token_lanes<LPT>(m, l, acc);

    if constexpr (WPP == 1) {
        if (!pair_ok || lt != 0)
            return;
        if (splits == 1) {
            const float inv = 1.0f / l;
            uint32_t h[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const _Float16 lo16 = (_Float16)(acc[2 * i] * inv);
                const _Float16 hi16 = (_Float16)(acc[2 * i + 1] * inv);
                h[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo16) | ((uint32_t)__builtin_bit_cast(uint16_t, hi16) << 16);
            }
            uint4 *dst = out + pc * (D / 8) + part * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[i] = make_uint4(h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]);
        } else {
            const int64_t item = (int64_t)split * pairs + pc;
            if (part == 0) {
                ws[item * 2] = m;
                ws[item * 2 + 1] = l;
            }
            float4 *dst = reinterpret_cast<float4 *>(ws + (int64_t)2 * splits * pairs + item * D + part * 32);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                dst[i] = make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
        }
    } else {
        if (lt == 0) {
#pragma unroll
            for (int i = 0; i < 32; ++i)
                sm_acc[wave][part * 32 + i] = acc[i];
            if (part == 0) {
                sm_ml[wave][0] = m;
                sm_ml[wave][1] = l;
            }
        }
        __syncthreads();
        if (wp != 0 || !pair_ok)
            return;
        const int w0 = pslot * WPP;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WPP; ++w)
            M = fmaxf(M, sm_ml[w0 + w][0]);
        const float Mr = (M == -INFINITY) ? 0.0f : M;
        float wt[WPP];
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < WPP; ++w) {
            wt[w] = exp2_fast(sm_ml[w0 + w][0] - Mr);
            L += wt[w] * sm_ml[w0 + w][1];
        }
        if (splits == 1) {
            const float inv = 1.0f / L;
            _Float16 *dst = reinterpret_cast<_Float16 *>(out) + pc * D;
#pragma unroll
            for (int j = 0; j < D / 64; ++j) {
                float o = 0.0f;
#pragma unroll
                for (int w = 0; w < WPP; ++w)
                    o += wt[w] * sm_acc[w0 + w][lane + 64 * j];
                dst[lane + 64 * j] = (_Float16)(o * inv);
            }
        } else {
            const int64_t item = (int64_t)split * pairs + pc;
            if (lane == 0) {
                ws[item * 2] = M;
                ws[item * 2 + 1] = L;
            }
            float *dst = ws + (int64_t)2 * splits * pairs + item * D;
#pragma unroll
            for (int j = 0; j < D / 64; ++j) {
                float o = 0.0f;
#pragma unroll
                for (int w = 0; w < WPP; ++w)
                    o += wt[w] * sm_acc[w0 + w][lane + 64 * j];
                dst[lane + 64 * j] = o;
            }
        }
    }
}

// Split-context reduce: one wave per (batch row, head).
//   M = max m_k,  L = sum 2^(m_k-M) l_k,  out = sum 2^(m_k-M) o_k / L
template <int D>
__global__ __launch_bounds__(256) void k_reduce(const float *__restrict__ ws, _Float16 *__restrict__ out, int pairs,
                                                int splits)
{
    const int lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= pairs)
        return;
    const float *__restrict__ accp = ws + (int64_t)2 * splits * pairs;
    float M = -INFINITY;
    for (int k = 0; k < splits; ++k)
        M = fmaxf(M, ws[((int64_t)k * pairs + pair) * 2]);
    const float Mr = (M == -INFINITY) ? 0.0f : M;
    float L = 0.0f;
    float o[D / 64];
#pragma unroll
    for (int j = 0; j < D / 64; ++j)
        o[j] = 0.0f;
    for (int k = 0; k < splits; ++k) {
        const int64_t item = (int64_t)k * pairs + pair;
        const float w = exp2_fast(ws[item * 2] - Mr);
        L += w * ws[item * 2 + 1];
#pragma unroll
        for (int j = 0; j < D / 64; ++j)
            o[j] += w * accp[item * D + lane + 64 * j];
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int j = 0; j < D / 64; ++j)
        out[pair * D + lane + 64 * j] = (_Float16)(o[j] * inv);
}

// ===========================================================================
// Top-k sparse decode attention.
//
// Contexts up to 2048 tokens: one kernel, k_topk_fused (below), scores in LDS.
// Longer contexts: two kernels.  k_topk_scores streams every key once (same
// lane layout and folded codec as k_decode; each wave takes a contiguous token
// range) and writes the scores, in log2 units, to a workspace of 4 bytes per
// token -- 5% of the key bytes.  k_topk_select then runs one 256-thread
// workgroup per (batch row, head): scores into LDS, the exact k-th largest by
// a 4-pass 8-bit radix select on order-preserving 32-bit keys, compaction of
// the kept tokens in ascending order (ties to the smaller index), softmax over
// the kept scores and P.V over their gathered V rows.
// ===========================================================================
__device__ __forceinline__ uint32_t order_key(float z)
{
    const uint32_t b = __builtin_bit_cast(uint32_t, z + 0.0f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes, in DPP moves (no LDS): row shifts
// by 1, 2, 4 and 8 inside each 16-lane row (lanes with no source add 0), then
// lane 15 of each row added to the next row (row_bcast:15, rows 1 and 3) and
// lane 31 to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int v, int /*lane*/)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true); // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true); // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true); // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true); // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31
    return v;
}

// The maximum (MAX) or minimum of v over the 64 lanes, in every lane: DPP
// exchanges inside each 16-lane row (xor 1, xor 2, mirror of 8, mirror of
// 16), then the row swaps across rows (permlane16 and permlane32).
template <bool MAX>
__device__ __forceinline__ float wave_extreme(float v)
{
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
    v = op(v, dpp<kQuadXor1>(v));
    v = op(v, dpp<kQuadXor2>(v));
    v = op(v, dpp<kHalfRowMirror>(v));
    v = op(v, dpp<0x140>(v)); // row_mirror: lane i <-> lane 15-i
    const auto r16 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                      false, false);
    v = op(__builtin_bit_cast(float, (uint32_t)r16[0]), __builtin_bit_cast(float, (uint32_t)r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                      false, false);
    return op(__builtin_bit_cast(float, (uint32_t)r32[0]), __builtin_bit_cast(float, (uint32_t)r32[1]));
}

// Exclusive prefix sum over the 256 threads of the block (in thread order).
__device__ __forceinline__ int block_excl_scan(int v, int *tmp4)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v, lane);
    if (lane == 63)
        tmp4[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w)
        base += tmp4[w];
    __syncthreads();
    return base + incl - v;
}

// The K rows of one score iteration (UU token rows per lane), clamped and
// flagged as in load_kv_rows.
template <int UU>
struct KRows {
    uint4 kx[UU];
    float km[UU], ks[UU];
};

template <int D, int UU, typename Meta>
__device__ __forceinline__ void load_k_rows(const CacheRow<Meta> &cr, int tb, int t_end, KRows<UU> &r)
{
    constexpr int TPW = 64 / (D / 32);
    constexpr int G = D / 64;
#pragma unroll
    for (int u = 0; u < UU; ++u) {
        const int t = tb + u * TPW;
        const uint32_t tcl = (uint32_t)(t < t_end ? t : t_end - 1);
        const uint32_t co = tcl * (D / 2) + cr.code_off, mo = tcl * (uint32_t)(sizeof(Meta) * G) + cr.meta_off;
        r.kx[u] = ld_stream16(cr.kb + co);
        r.km[u] = ld_meta(at_byte(cr.kmb, mo));
        r.ks[u] = ld_meta(at_byte(cr.ksb, mo));
    }
}

// Every lane of a token row holds the row's score after token_sum, so lane
// `part` of each row stores rows u = part, part + LPT, ...: at d = 128 one
// nontemporal store instruction writes all 64 rows of a 4-row iteration (256
// contiguous bytes).  The scores' writes, mixed into the key stream, cost the
// pass ~12% of its read rate; long nontemporal runs cost the least (measured:
// 83.6 us against 85.8 us with 64-byte runs by a quarter of the lanes and
// 87.3 us with ordinary stores).
template <int D, int UU>
__device__ __forceinline__ void store_scores(const KRows<UU> &r, int tb, int t_end, const QSlice &qs, const Magic mg,
                                             float c2, int part, float *__restrict__ srow)
{
    constexpr int LPT = D / 32;
    constexpr int TPW = 64 / LPT;
    float zs[UU];
#pragma unroll
    for (int u = 0; u < UU; ++u) {
        const float dq = dot_keys(qs, r.kx[u], mg);
        const float sp = __builtin_fmaf(r.ks[u], dq, r.km[u] * qs.qsum);
        zs[u] = token_sum<LPT>(sp) * c2;
    }
#pragma unroll
    for (int i = 0; i < (UU + LPT - 1) / LPT; ++i) {
        const int u = part + i * LPT; // this lane's row of the iteration
        float z = zs[0];
#pragma unroll
        for (int uu = 1; uu < UU; ++uu)
            z = u == uu ? zs[uu] : z;
        const int t = tb + u * TPW;
        if (u < UU && t < t_end)
            __builtin_nontemporal_store(z, srow + t);
    }
}

template <int D, int UU, typename Meta>
__device__ __forceinline__ void score_iter(const CacheRow<Meta> &cr, int tb, int t_end, const QSlice &qs, const Magic mg,
                                           float c2, int part, float *__restrict__ srow)
{
    KRows<UU> r;
    load_k_rows<D, UU>(cr, tb, t_end, r);
    store_scores<D, UU>(r, tb, t_end, qs, mg, c2, part, srow);
}

// One wave per (pair, chunk of `chunk` tokens); four waves per workgroup.
template <int D, int U, typename Meta>
__global__ __launch_bounds__(256) void k_topk_scores(const uint8_t *__restrict__ kc, const Meta *__restrict__ kmin,
                                                     const Meta *__restrict__ ksc, const uint4 *__restrict__ q,
                                                     float *__restrict__ scores, int pairs, int S, int T,
                                                     int chunk, int n_chunks, float c2)
{
    constexpr int LPT = D / 32;
    constexpr int TPW = 64 / LPT;
    constexpr int TPI = U * TPW;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (int64_t)pairs * n_chunks)
        return;
    const int64_t pair = item / n_chunks;
    const int c = (int)(item - pair * n_chunks);
    const int part = lane % LPT, lt = lane / LPT;
    const int w_begin = c * chunk;
    const int t_end = min(T, w_begin + chunk);
    const int n_full = (t_end - w_begin) / TPI;
    const int n_rest = (t_end - w_begin - n_full * TPI + TPW - 1) / TPW;
    const CacheRow<Meta> cr = cache_row<D, Meta>(kc, nullptr, kmin, ksc, nullptr, nullptr, (int)pair, S, part);
    float *__restrict__ srow = scores + pair * T;
    int tb = w_begin + lt;
    // the first iteration's rows are requested right behind the query
    const QRaw qraw = load_q_raw(q + pair * (D / 8) + part * 4);
    KRows<U> first;
    if (n_full > 0)
        load_k_rows<D, U>(cr, tb, t_end, first);
    const QSlice qs = q_slice(qraw);
    const Magic mg = magic_vgprs();
    if (n_full > 0) {
        store_scores<D, U>(first, tb, t_end, qs, mg, c2, part, srow);
        tb += TPI;
    }
    for (int it = 1; it < n_full; ++it, tb += TPI)
        score_iter<D, U>(cr, tb, t_end, qs, mg, c2, part, srow);
    for (int it = 0; it < n_rest; ++it, tb += TPW)
        score_iter<D, 1>(cr, tb, t_end, qs, mg, c2, part, srow);
}

template <int D, typename Meta>
__global__ __launch_bounds__(256) void k_topk_select(const uint8_t *__restrict__ vc, const Meta *__restrict__ vmin,
                                                     const Meta *__restrict__ vsc, const float *__restrict__ scores,
                                                     _Float16 *__restrict__ out, int32_t *__restrict__ sel_out,
                                                     int S, int T, int k_top)
{
    constexpr int LPT = D / 32;
    constexpr int TPW = 64 / LPT;
    constexpr int G = D / 64;
    constexpr int UG = 4; // gathered rows per lane in flight
    extern __shared__ __attribute__((aligned(16))) float sm_dyn[];
    float *__restrict__ sc = sm_dyn;                                        // [T] scores, log2 units
    uint16_t *__restrict__ sel = reinterpret_cast<uint16_t *>(sm_dyn + T);  // [k_top] kept tokens
    __shared__ int hist[256];
    __shared__ int tmp4[4];
    __shared__ float red[4];
    __shared__ float sm_acc[4][D];
    __shared__ int sh_digit, sh_above;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t pair = blockIdx.x;
    const int part = lane % LPT, lt = lane / LPT, g = part >> 1;

    // (1) scores into LDS, and their maximum: 16-byte loads, up to four per
    // thread in flight (the row of T floats is 16-byte aligned when T % 4 == 0;
    // otherwise, and for the tail, single floats)
    const float *__restrict__ srow = scores + pair * T;
    float zmax = -INFINITY;
    const int T4 = (T % 4 == 0) ? T / 4 : 0;
    for (int i0 = tid; i0 < T4; i0 += 256 * 4) {
        // clamped indices: a lane past the end reloads (and rewrites, with the
        // same value) the last float4, so no load sits behind a branch
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = ld_stream16(srow + 4 * min(i0 + u * 256, T4 - 1));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float z0 = __builtin_bit_cast(float, v[u].x), z1 = __builtin_bit_cast(float, v[u].y);
            const float z2 = __builtin_bit_cast(float, v[u].z), z3 = __builtin_bit_cast(float, v[u].w);
            reinterpret_cast<float4 *>(sc)[min(i0 + u * 256, T4 - 1)] = make_float4(z0, z1, z2, z3);
            zmax = fmaxf(zmax, fmaxf(fmaxf(z0, z1), fmaxf(z2, z3)));
        }
    }
    for (int t = 4 * T4 + tid; t < T; t += 256) {
        const float z = ld_stream(srow + t);
        sc[t] = z;
        zmax = fmaxf(zmax, z);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        zmax = fmaxf(zmax, __shfl_xor(zmax, off));
    if (lane == 0)
        red[wave] = zmax;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

    // (2) radix select of the k_top-th largest key
    uint32_t prefix = 0, pmask = 0;
    int remaining = k_top;
    for (int shift = 24; shift >= 0; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
        for (int t = tid; t < T; t += 256) {
            const uint32_t key = order_key(sc[t]);
            if ((key & pmask) == prefix)
                atomicAdd(&hist[(key >> shift) & 255], 1);
        }
        __syncthreads();
        const int cnt = hist[255 - tid];                // thread i looks at digit 255-i
        const int before = block_excl_scan(cnt, tmp4);  // keys with a larger digit
        if (before < remaining && remaining <= before + cnt) {
            sh_digit = 255 - tid;
            sh_above = before;
        }
        __syncthreads();
        prefix |= (uint32_t)sh_digit << shift;
        pmask |= 255u << shift;
        remaining -= sh_above;
        __syncthreads();
    }
    const uint32_t thr = prefix; // exact key of the k_top-th largest score
    // `remaining` keys equal to thr are kept: the ones with the smallest index.

    // (3) compaction in ascending token order: thread tid owns a contiguous chunk
    const int chunk = (T + 255) / 256;
    const int c0 = min(T, tid * chunk), c1 = min(T, c0 + chunk);
    int neq = 0;
    for (int t = c0; t < c1; ++t)
        neq += order_key(sc[t]) == thr;
    const int eq_before = block_excl_scan(neq, tmp4);
    int nsel = 0;
    {
        int e = eq_before;
        for (int t = c0; t < c1; ++t) {
            const uint32_t key = order_key(sc[t]);
            const bool keep = key > thr || (key == thr && e < remaining);
            e += key == thr;
            nsel += keep;
        }
    }
    int pos = block_excl_scan(nsel, tmp4);
    {
        int e = eq_before;
        for (int t = c0; t < c1; ++t) {
            const uint32_t key = order_key(sc[t]);
            const bool keep = key > thr || (key == thr && e < remaining);
            e += key == thr;
            if (keep)
                sel[pos++] = (uint16_t)t;
        }
    }
    __syncthreads();

    // (4) softmax over the kept scores and P.V over their V rows, UG rows per
    // lane in flight
    const uint8_t *__restrict__ vb = vc + pair * S * (D / 2) + part * 16;
    const Meta *__restrict__ vmb = vmin + pair * S * G + g;
    const Meta *__restrict__ vsb = vsc + pair * S * G + g;
    float l = 0.0f, bsum = 0.0f;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i)
        acc[i] = 0.0f;
    for (int j0 = wave * TPW + lt; j0 < k_top; j0 += 4 * TPW * UG) {
        uint4 vx[UG];
        float vm[UG], vs[UG], p[UG];
#pragma unroll
        for (int u = 0; u < UG; ++u) {
            const int j = j0 + u * 4 * TPW;
            const bool valid = j < k_top;
            const int64_t t = sel[valid ? j : k_top - 1];
            vx[u] = ld_stream16(vb + t * (D / 2));
            vm[u] = ld_meta(vmb + t * G);
            vs[u] = ld_meta(vsb + t * G);
            p[u] = valid ? exp2_fast(sc[t] - M) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < UG; ++u) {
            l += p[u];
            bsum = __builtin_fmaf(p[u], vm[u], bsum);
            axpy_values(acc, p[u] * (vs[u] * kTwo24), vx[u]);
        }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i)
        acc[i] += bsum;
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
        l += __shfl_xor(l, off);
#pragma unroll
        for (int i = 0; i < 32; ++i)
            acc[i] += __shfl_xor(acc[i], off);
    }
    if (lt == 0) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
            sm_acc[wave][part * 32 + i] = acc[i];
        if (part == 0)
            red[wave] = l;
    }
    __syncthreads();
    const float L = red[0] + red[1] + red[2] + red[3];
    const float inv = 1.0f / L;
    for (int i = tid; i < D; i += 256)
        out[pair * D + i] = (_Float16)((sm_acc[0][i] + sm_acc[1][i] + sm_acc[2][i] + sm_acc[3][i]) * inv);
    if (sel_out != nullptr)
        for (int j = tid; j < k_top; j += 256)
            sel_out[pair * k_top + j] = sel[j];
}

// Contexts up to 2048 tokens: the whole call in one launch, one workgroup of
// NWV waves (1, 2 or 4) per (batch row, head).
//  (1) Scores: wave w streams the keys of the w-th of NWV equal parts of the
//      context (the lane layout and folded codec of k_decode) and writes each
//      score into LDS, transposed so that lane l of wave 0 can then hold the
//      keys of the KPL consecutive tokens KPL*l .. KPL*l+KPL-1 in registers
//      (KPL = 16 for contexts up to 1024, else 32); ascending token order is
//      then lane-major order.  The scores go to the workspace as well when one
//      is given.
//  (2) Threshold and compaction, by wave 0 alone.  The threshold (the
//      k_top-th largest key) is found in two levels.  A 256-bin histogram of
//      the scores over [min, max] (LDS atomics; the bin is a monotone function
//      of the score, so every key in a higher bin is larger) gives the bin b*
//      that holds the k_top-th largest key and the number A of keys in higher
//      bins.  The keys of bin b* (at most 64, one per lane) are then searched
//      bit by bit for their (k_top - A)-th largest: the largest v with at
//      least k_top - A of them >= v.  When bin b* holds more than 64 keys
//      (scores crowded into a narrow range), the same bit-by-bit search runs
//      over all the keys instead.  A search step that finds exactly the wanted
//      count has found the selection itself and stops early.  One prefix sum
//      over the lanes then places each lane's kept tokens (ties to the smaller
//      index); their indices and softmax weights go to LDS.
//  (3) P.V: the waves gather the kept V rows in rounds of TPW * UG rows, UG
//      rows per lane in flight; with NWV > 1 their partial sums are added in
//      LDS.
// The scores never leave the chip, and while one wave selects, the other
// waves resident on its compute unit keep streaming keys.  One wave per pair
// needs no workgroup barrier and leaves no wave idle during the selection;
// two or four share a pair when there are too few pairs to fill the compute
// units that way.
// v <- sum of v over the lanes congruent to this one modulo STEP (STEP a power
// of two, 2..32): row rotations by STEP, 2 STEP, .. 8 inside each 16-lane row
// (DPP, no LDS), then exchanges across rows.
template <int STEP>
__device__ __forceinline__ void lane_group_sum(float &v)
{
#pragma unroll
    for (int off = STEP; off < 16; off <<= 1)
        v += off == 1 ? dpp<0x121>(v) : off == 2 ? dpp<0x122>(v) : off == 4 ? dpp<0x124>(v) : dpp<0x128>(v);
#pragma unroll
    for (int off = STEP < 16 ? 16 : STEP; off < 64; off <<= 1)
        v += __shfl_xor(v, off);
}

// Inverse of order_key.
__device__ __forceinline__ float tr_key_to_z(uint32_t kb)
{
    return __builtin_bit_cast(float, (kb & 0x80000000u) ? (kb ^ 0x80000000u) : ~kb);
}

// 0 <= (z - zmin) * bscale <= 256 (1 + 2^-22) for zmin <= z <= zmax.
__device__ __forceinline__ int key_bin(uint32_t kb, float zmin, float bscale)
{
    return (int)fminf((tr_key_to_z(kb) - zmin) * bscale, 255.0f);
}

__device__ __forceinline__ int wave_sum_small(int c) // 0 <= c < 64 in every lane
{
    int s = 0;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit)
        s += __popcll(__ballot((c >> bit) & 1)) << bit;
    return s;
}

// The largest v such that at least `want` of the wave's keys (key_at(0) ..
// key_at(N-1) in each lane) are >= v: the want-th largest key.  With EARLY, a
// candidate that has exactly `want` keys >= it ends the search, returning that
// candidate minus one (the keys > the result are then exactly the wanted
// ones); this is only valid when the keys searched are all the keys.  Keys of
// 0 never count: every candidate is >= 1.
template <int N, bool EARLY, typename KeyAt>
__device__ __forceinline__ uint32_t greedy_threshold(KeyAt key_at, int want)
{
    uint32_t thr = 0;
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = thr | (1u << b);
        int cnt;
        if constexpr (N == 1) {
            cnt = __popcll(__ballot(key_at(0) >= cand));
        } else {
            int c = 0;
#pragma unroll
            for (int i = 0; i < N; ++i)
                c += key_at(i) >= cand;
            cnt = wave_sum_small(c);
        }
        if (cnt >= want) {
            thr = cand;
            if (EARLY && cnt == want)
                return cand - 1u;
        }
    }
    return thr;
}

// Scores of one iteration's rows into the transposed LDS layout (and into
// srow when it is given): every lane of a token row holds the row's score
// after token_sum, lane `part` writes rows u = part, part + LPT, ...
template <int D, int UU, int KPL>
__device__ __forceinline__ void put_scores(const KRows<UU> &r, int tb, int t_end, const QSlice &qs, const Magic mg,
                                           float c2, int part, float *__restrict__ tr, float *__restrict__ srow)
{
    constexpr int LPT = D / 32;
    constexpr int TPW = 64 / LPT;
    float zs[UU];
#pragma unroll
    for (int u = 0; u < UU; ++u) {
        const float dq = dot_keys(qs, r.kx[u], mg);
        const float sp = __builtin_fmaf(r.ks[u], dq, r.km[u] * qs.qsum);
        zs[u] = token_sum<LPT>(sp) * c2;
    }
#pragma unroll
    for (int i = 0; i < (UU + LPT - 1) / LPT; ++i) {
        const int u = part + i * LPT; // this lane's row of the iteration
        float z = zs[0];
#pragma unroll
        for (int uu = 1; uu < UU; ++uu)
            z = u == uu ? zs[uu] : z;
        const int t = tb + u * TPW;
        if (u < UU && t < t_end) {
            tr[(t / KPL) * (KPL + 1) + t % KPL] = z;
            if (srow != nullptr)
                __builtin_nontemporal_store(z, srow + t);
        }
    }
}

template <int D, int UU, int KPL, typename Meta>
__device__ __forceinline__ void score_iter_lds(const CacheRow<Meta> &cr, int tb, int t_end, const QSlice &qs,
                                               const Magic mg, float c2, int part, float *__restrict__ tr,
                                               float *__restrict__ srow)
{
    KRows<UU> r;
    load_k_rows<D, UU>(cr, tb, t_end, r);
    put_scores<D, UU, KPL>(r, tb, t_end, qs, mg, c2, part, tr, srow);
}

// Dynamic LDS: the transposed scores [64][KPL + 1]; the waves' partial sums
// [4][D] and their softmax sums [4]; then `region_bytes` for wave 0's
// histogram [256] (+64 discard counters) and bin b*'s keys [64] (+64 discard
// slots), later the kept tokens' scores relative to the maximum and their
// indices [k_top] (+64 discard slots each).
template <int D, int NWV, int U, int KPL, int UG, typename Meta>
__global__ __launch_bounds__(64 * NWV) void k_topk_fused(const uint8_t *__restrict__ kc, const Meta *__restrict__ kmin,
                                                    const Meta *__restrict__ ksc, const uint8_t *__restrict__ vc,
                                                    const Meta *__restrict__ vmin, const Meta *__restrict__ vsc,
                                                    const uint4 *__restrict__ q, float *__restrict__ scores,
                                                    _Float16 *__restrict__ out, int32_t *__restrict__ sel_out, int S,
                                                    int T, int k_top, int part_len, float c2)
{
    constexpr int LPT = D / 32;
    constexpr int TPW = 64 / LPT;
    constexpr int TPI = U * TPW;
    constexpr int G = D / 64;
    constexpr int ROW = KPL + 1; // LDS row of one lane's keys, padded against bank conflicts
    extern __shared__ __attribute__((aligned(16))) float sm_dyn[];
    float *__restrict__ tr = sm_dyn;
    float *__restrict__ red = sm_dyn + 64 * ROW; // [NWV][D], then the NWV sums
    char *__restrict__ region = reinterpret_cast<char *>(red + NWV * D + 4);
    int *__restrict__ hist = reinterpret_cast<int *>(region);
    uint32_t *__restrict__ cand = reinterpret_cast<uint32_t *>(region + 4 * (256 + 64));
    float *__restrict__ sel_z = reinterpret_cast<float *>(region);
    uint16_t *__restrict__ sel_t = reinterpret_cast<uint16_t *>(region + 4 * (size_t)(k_top + 64));

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t pair = blockIdx.x;
    const int part = lane % LPT, lt = lane / LPT;

    // (1) scores of the wave's part of the context
    {
        const int w_begin = wave * part_len;
        const int t_end = min(T, w_begin + part_len);
        if (t_end > w_begin) {
            const int n_full = (t_end - w_begin) / TPI;
            const int n_rest = (t_end - w_begin - n_full * TPI + TPW - 1) / TPW;
            const CacheRow<Meta> cr = cache_row<D, Meta>(kc, nullptr, kmin, ksc, nullptr, nullptr, (int)pair, S, part);
            float *__restrict__ srow = scores != nullptr ? scores + pair * T : nullptr;
            int tb = w_begin + lt;
            // the first iteration's rows are requested right behind the query
            const QRaw qraw = load_q_raw(q + pair * (D / 8) + part * 4);
            KRows<U> first;
            if (n_full > 0)
                load_k_rows<D, U>(cr, tb, t_end, first);
            const QSlice qs = q_slice(qraw);
            const Magic mg = magic_vgprs();
            if (n_full > 0) {
                put_scores<D, U, KPL>(first, tb, t_end, qs, mg, c2, part, tr, srow);
                tb += TPI;
            }
            for (int it = 1; it < n_full; ++it, tb += TPI)
                score_iter_lds<D, U, KPL>(cr, tb, t_end, qs, mg, c2, part, tr, srow);
            for (int it = 0; it < n_rest; ++it, tb += TPW)
                score_iter_lds<D, 1, KPL>(cr, tb, t_end, qs, mg, c2, part, tr, srow);
        }
    }
    __syncthreads();

    // (2) threshold and compaction (wave 0)
    if (wave == 0) {
        // lane l: tokens KPL*l .. KPL*l+KPL-1; keys of t >= T are 0, below every
        // finite score's key
        uint32_t key[KPL];
        float zmax = -INFINITY, zmin = INFINITY;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const float z = tr[lane * ROW + i];
            const bool valid = KPL * lane + i < T;
            zmax = fmaxf(zmax, valid ? z : -INFINITY);
            zmin = fminf(zmin, valid ? z : INFINITY);
            key[i] = valid ? order_key(z) : 0u;
        }
        zmax = wave_extreme<true>(zmax);
        zmin = wave_extreme<false>(zmin);

        // Bins: bin(z) = (int)min((z - zmin) * bscale, 255), monotone in z; a
        // zero (or unrepresentable) range gives one bin and the full search.
        // No branch: the keys of t >= T count in their lane's own discard counter.
        const float zrange = zmax - zmin;
        const float bscale = (zrange > 1e-30f && zrange <= 3e38f) ? 256.0f / zrange : 0.0f;
        reinterpret_cast<int4 *>(hist)[lane] = make_int4(0, 0, 0, 0); // the discard counters are never read
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        uint32_t bins[KPL / 4]; // four 8-bit bins per register
#pragma unroll
        for (int r = 0; r < KPL / 4; ++r)
            bins[r] = 0u;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const int bi = key_bin(key[i], zmin, bscale);
            bins[i / 4] |= (uint32_t)bi << (8 * (i % 4));
            atomicAdd(&hist[key[i] != 0u ? bi : 256 + lane], 1);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        // counts of the keys in bins >= b, from the top: lane l holds bins 4l..4l+3
        const int4 h4 = reinterpret_cast<const int4 *>(hist)[lane];
        const int lsum = h4.x + h4.y + h4.z + h4.w;
        const int lincl = wave_incl_scan(lsum, lane);
        const int above_lane = __builtin_amdgcn_readlane(lincl, 63) - lincl; // keys in bins of higher lanes
        const int ge3 = above_lane + h4.w, ge2 = ge3 + h4.z, ge1 = ge2 + h4.y, ge0 = ge1 + h4.x;
        // bin b* holds the k_top-th largest: ge(b*+1) < k_top <= ge(b*)
        int my_bin = -1, my_above = 0, my_n = 0;
        if (above_lane < k_top && k_top <= ge3) { my_bin = 4 * lane + 3; my_above = above_lane; my_n = h4.w; }
        if (ge3 < k_top && k_top <= ge2) { my_bin = 4 * lane + 2; my_above = ge3; my_n = h4.z; }
        if (ge2 < k_top && k_top <= ge1) { my_bin = 4 * lane + 1; my_above = ge2; my_n = h4.y; }
        if (ge1 < k_top && k_top <= ge0) { my_bin = 4 * lane; my_above = ge1; my_n = h4.x; }
        const uint64_t owner = __ballot(my_bin >= 0);
        const int src = (int)__builtin_ctzll(owner);
        const int bstar = __builtin_amdgcn_readlane(my_bin, src), n_star = __builtin_amdgcn_readlane(my_n, src),
                  a_star = __builtin_amdgcn_readlane(my_above, src);
        uint32_t thr;
        if (n_star <= 64) {
            // bin b*'s keys, one per lane; the others go to discard slots
            int c = 0;
#pragma unroll
            for (int i = 0; i < KPL; ++i)
                c += (key[i] != 0u) & ((int)((bins[i / 4] >> (8 * (i % 4))) & 255u) == bstar);
            int p = wave_incl_scan(c, lane) - c;
#pragma unroll
            for (int i = 0; i < KPL; ++i) {
                const bool in = (key[i] != 0u) & ((int)((bins[i / 4] >> (8 * (i % 4))) & 255u) == bstar);
                cand[in ? p : 64 + lane] = key[i];
                p += in;
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            const uint32_t ck = lane < n_star ? cand[lane] : 0u;
            // an exact key: lower bins stay below
            thr = greedy_threshold<1, false>([&](int) { return ck; }, k_top - a_star);
        } else {
            thr = greedy_threshold<KPL, true>([&](int i) { return key[i]; }, k_top);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier(); // hist and cand are read before sel_z/sel_t reuse the region

        // compaction in ascending token order: one prefix sum over the lanes of
        // (keys > thr) and (keys == thr); the first `remaining` keys equal to thr
        // (smallest indices) are kept.  Dropped keys write to discard slots.
        int gt = 0, eq = 0;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            gt += key[i] > thr;
            eq += key[i] == thr;
        }
        const int packed = gt | (eq << 16);
        const int incl = wave_incl_scan(packed, lane);
        const int tot = __builtin_amdgcn_readlane(incl, 63);
        const int excl = incl - packed;
        const int remaining = k_top - (tot & 0xFFFF);
        int eq_rank = excl >> 16;
        int pos = (excl & 0xFFFF) + min(eq_rank, remaining);
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const uint32_t kb = key[i];
            const bool is_eq = kb == thr;
            const bool keep = (kb > thr) | (is_eq & (eq_rank < remaining));
            eq_rank += is_eq;
            const int slot = keep ? pos : k_top + lane;
            sel_z[slot] = tr_key_to_z(kb) - zmax;
            sel_t[slot] = (uint16_t)(KPL * lane + i);
            pos += keep;
        }
    }
    __syncthreads();

    // (3) P.V over the kept rows: wave w takes rounds w, w + NWV, .. of TPW * UG
    // rows, UG rows per lane in flight
    const CacheRow<Meta> cv = cache_row<D, Meta>(nullptr, vc, nullptr, nullptr, vmin, vsc, (int)pair, S, part);
    float l = 0.0f, bsum = 0.0f;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i)
        acc[i] = 0.0f;
    for (int j0 = wave * (TPW * UG); j0 < k_top; j0 += NWV * (TPW * UG)) {
        uint4 vx[UG];
        float vm[UG], vs[UG], p[UG];
#pragma unroll
        for (int u = 0; u < UG; ++u) {
            const int j = j0 + u * TPW + lt;
            const int jc = min(j, k_top - 1);
            const uint32_t t = sel_t[jc];
            vx[u] = ld_stream16(cv.vb + (t * (D / 2) + cv.code_off));
            vm[u] = ld_meta(at_byte(cv.vmb, t * (uint32_t)(sizeof(Meta) * G) + cv.meta_off));
            vs[u] = ld_meta(at_byte(cv.vsb, t * (uint32_t)(sizeof(Meta) * G) + cv.meta_off));
            p[u] = j < k_top ? exp2_fast(sel_z[jc]) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < UG; ++u) {
            l += p[u];
            bsum = __builtin_fmaf(p[u], vm[u], bsum);
            axpy_values(acc, p[u] * (vs[u] * kTwo24), vx[u]);
        }
    }
    if (sel_out != nullptr)
        for (int j = tid; j < k_top; j += 64 * NWV)
            sel_out[pair * k_top + j] = sel_t[j];
#pragma unroll
    for (int i = 0; i < 32; ++i)
        acc[i] += bsum;
    // sum over the token lanes (lanes of equal `part`): rotations inside each
    // 16-lane row (DPP), then across rows; then over the NWV waves in LDS
    lane_group_sum<LPT>(l);
#pragma unroll
    for (int i = 0; i < 32; ++i)
        lane_group_sum<LPT>(acc[i]);
    if (lt == 0) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
            red[wave * D + 32 * part + i] = acc[i];
        if (part == 0)
            red[NWV * D + wave] = l;
    }
    __syncthreads();
    if (wave == 0) {
        float lsum = red[NWV * D];
#pragma unroll
        for (int w = 1; w < NWV; ++w)
            lsum += red[NWV * D + w];
        const float inv = 1.0f / lsum;
#pragma unroll
        for (int e = 0; e < D / 64; ++e) {
            const int i = lane * (D / 64) + e;
            float o = red[i];
#pragma unroll
            for (int w = 1; w < NWV; ++w)
                o += red[w * D + i];
            out[pair * D + i] = (_Float16)(o * inv);
        }
    }
}

// ===========================================================================
// Read-only HBM stream (the measured ceiling the attention kernels are held
// to): each lane reads 16 consecutive 16-byte pieces (a workgroup 64 KB)
// with the same nontemporal 16-byte loads as the cache streams, all in
// flight together, and folds them into one word.  The only store is guarded
// by a value the data never reaches in practice, so it keeps the loads
// live without writing memory.
// ===========================================================================
__global__ __launch_bounds__(256) void k_stream_read(const uint4 *__restrict__ p, int64_t n16,
                                                     uint32_t *__restrict__ sink)
{
    constexpr int U = 16;
    const int64_t base = (int64_t)blockIdx.x * (256 * U) + threadIdx.x;
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        v[u] = ld_stream16(p + min(base + (int64_t)u * 256, n16 - 1));
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
        acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (acc == 0x9E3779B9u)
        sink[blockIdx.x] = acc;
}

// ---------------------------------------------------------------------------
template <typename Meta>
Meta *meta(void *p)
{
    return static_cast<Meta *>(p);
}

template <int D, typename Meta>
int launch_quantize_d(const CachePlanes &c, const void *k, const void *v, int b, int s_src, int t_dst0,
                      hipStream_t st)
{
    constexpr int RPB = 256 / (D / 8);
    const int pairs = b * c.a; // < 2^31: checked with the cache dimensions
    auto *kc = reinterpret_cast<uint32_t *>(c.k_codes);
    auto *vc = reinterpret_cast<uint32_t *>(c.v_codes);
    const auto *ks = static_cast<const uint4 *>(k);
    const auto *vs = static_cast<const uint4 *>(v);
    const FastDiv by_a = make_fast_div((uint32_t)c.a);
    if (s_src == 1) {
        const dim3 grid((unsigned)((pairs + RPB - 1) / RPB), 2);
        hipLaunchKernelGGL((k_quantize<D, 1, Meta>), grid, dim3(256), 0, st, ks, vs, pairs, 1, 1, make_fast_div(1),
                           c.a, by_a, c.S, t_dst0, kc, vc, meta<Meta>(c.k_min), meta<Meta>(c.k_scale),
                           meta<Meta>(c.v_min), meta<Meta>(c.v_scale));
    } else {
        // two rows per thread: measured against four on the OPT-175B, OPT-30B and
        // OPT-6.7B prompts, 1.7 %, 0.6 % and 3.9 % faster (eight: 12-15 % slower)
        constexpr int R = 2;
        const int chunks = (s_src + RPB * R - 1) / (RPB * R);
        const int64_t blocks = (int64_t)pairs * chunks;
        if (blocks > 0x7FFFFFFF)
            return (int)hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((k_quantize<D, R, Meta>), dim3((unsigned)blocks, 2), dim3(256), 0, st, ks, vs, pairs,
                           s_src, chunks, make_fast_div((uint32_t)chunks), c.a, by_a, c.S, t_dst0, kc, vc,
                           meta<Meta>(c.k_min), meta<Meta>(c.k_scale), meta<Meta>(c.v_min), meta<Meta>(c.v_scale));
    }
    return (int)hipGetLastError();
}

template <int D, int U, int WPP, typename Meta>
int launch_decode_k(const CachePlanes &c, int pairs, const void *q, int T, void *out, const DecodeShape &sh,
                    float *ws, const void *k_new, const void *v_new, hipStream_t st)
{
    constexpr int PPB = 4 / WPP;
    const float c2 = 1.4426950408889634f / sqrtf((float)D);
    const int64_t blocks = (int64_t)((pairs + PPB - 1) / PPB) * sh.splits;
    hipLaunchKernelGGL((k_decode<D, U, WPP, Meta>), dim3((unsigned)blocks), dim3(256), 0, st, c.k_codes, c.v_codes,
                       meta<Meta>(c.k_min), meta<Meta>(c.k_scale), meta<Meta>(c.v_min), meta<Meta>(c.v_scale),
                       static_cast<const uint4 *>(q),
                       static_cast<uint4 *>(out), ws, pairs, c.S, T, sh.splits, sh.split_len, c2,
                       static_cast<const uint4 *>(k_new), static_cast<const uint4 *>(v_new));
    int e = (int)hipGetLastError();
    if (e != 0 || sh.splits == 1)
        return e;
    hipLaunchKernelGGL((k_reduce<D>), dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, st, ws,
                       static_cast<_Float16 *>(out), pairs, sh.splits);
    return (int)hipGetLastError();
}

template <int D, int U, typename Meta>
int launch_decode_u(const CachePlanes &c, int pairs, const void *q, int T, void *out, const DecodeShape &sh,
                    float *ws, const void *k_new, const void *v_new, hipStream_t st)
{
    switch (sh.waves_per_pair) {
    case 1: return launch_decode_k<D, U, 1, Meta>(c, pairs, q, T, out, sh, ws, k_new, v_new, st);
    case 2: return launch_decode_k<D, U, 2, Meta>(c, pairs, q, T, out, sh, ws, k_new, v_new, st);
    default: return launch_decode_k<D, U, 4, Meta>(c, pairs, q, T, out, sh, ws, k_new, v_new, st);
    }
}

template <int D, typename Meta>
int launch_decode_d(const CachePlanes &c, int pairs, const void *q, int T, void *out, const DecodeShape &sh,
                    float *ws, const void *k_new, const void *v_new, hipStream_t st)
{
    switch (sh.unroll) {
    case 1: return launch_decode_u<D, 1, Meta>(c, pairs, q, T, out, sh, ws, k_new, v_new, st);
    case 2: return launch_decode_u<D, 2, Meta>(c, pairs, q, T, out, sh, ws, k_new, v_new, st);
    default: return launch_decode_u<D, 4, Meta>(c, pairs, q, T, out, sh, ws, k_new, v_new, st);
    }
}

constexpr int kTopkCUs = 256; // compute units of MI355X

// k_topk_fused with NWV waves per pair: U = 8 key rows per lane in flight,
// UG gathered V rows per lane chosen so that one round of the waves covers at
// least 208 rows at head_dim 128 (the top 10% of contexts up to 2080).
template <int D, int NWV, int KPL, typename Meta>
int launch_topk_fused(const CachePlanes &c, int pairs, const void *q, int T, int k_top, void *out, int32_t *sel,
                      float *ws, float c2, hipStream_t st)
{
    constexpr int TPW = 64 / (D / 32);
    constexpr int UG = NWV == 1 ? 13 : NWV == 2 ? 7 : 4;
    const int part = ((T + NWV - 1) / NWV + TPW - 1) / TPW * TPW; // tokens per wave
    const size_t sel_bytes = (size_t)(k_top + 64) * (sizeof(float) + sizeof(uint16_t));
    const size_t region = (std::max(sel_bytes, (size_t)4 * (256 + 64 + 128)) + 15) / 16 * 16;
    const size_t lds = (size_t)4 * (64 * (KPL + 1) + NWV * D + 4) + region;
    hipLaunchKernelGGL((k_topk_fused<D, NWV, 8, KPL, UG, Meta>), dim3((unsigned)pairs), dim3(64 * NWV), lds, st,
                       c.k_codes, meta<Meta>(c.k_min), meta<Meta>(c.k_scale), c.v_codes, meta<Meta>(c.v_min),
                       meta<Meta>(c.v_scale), static_cast<const uint4 *>(q), ws, static_cast<_Float16 *>(out), sel, c.S,
                       T, k_top, part, c2);
    return (int)hipGetLastError();
}

template <int D, typename Meta>
int launch_topk_d(const CachePlanes &c, int pairs, const void *q, int T, int k_top, void *out, int32_t *sel,
                  float *ws, hipStream_t st)
{
    constexpr int TPW = 64 / (D / 32);
    const float c2 = 1.4426950408889634f / sqrtf((float)D);
    if (T <= KVQ_TOPK_FUSED_MAX_CTX) {
        // waves per pair: one when the pairs alone give every compute unit 12
        // waves (three per SIMD, the occupancy of these kernels), else two or
        // four (measured on MI355X at 768 .. 6144 pairs)
        const int nwv = pairs >= 12 * kTopkCUs ? 1 : pairs >= 3 * kTopkCUs ? 2 : 4;
        if (T <= 1024) {
            switch (nwv) {
            case 1: return launch_topk_fused<D, 1, 16, Meta>(c, pairs, q, T, k_top, out, sel, ws, c2, st);
            case 2: return launch_topk_fused<D, 2, 16, Meta>(c, pairs, q, T, k_top, out, sel, ws, c2, st);
            default: return launch_topk_fused<D, 4, 16, Meta>(c, pairs, q, T, k_top, out, sel, ws, c2, st);
            }
        }
        switch (nwv) {
        case 1: return launch_topk_fused<D, 1, 32, Meta>(c, pairs, q, T, k_top, out, sel, ws, c2, st);
        case 2: return launch_topk_fused<D, 2, 32, Meta>(c, pairs, q, T, k_top, out, sel, ws, c2, st);
        default: return launch_topk_fused<D, 4, 32, Meta>(c, pairs, q, T, k_top, out, sel, ws, c2, st);
        }
    }
    const int chunk = std::min(128, (T + TPW - 1) / TPW * TPW);
    const int n_chunks = (T + chunk - 1) / chunk;
    const int64_t waves = (int64_t)pairs * n_chunks;
    hipLaunchKernelGGL((k_topk_scores<D, 4, Meta>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, c.k_codes,
                       meta<Meta>(c.k_min), meta<Meta>(c.k_scale), static_cast<const uint4 *>(q), ws, pairs, c.S, T, chunk, n_chunks, c2);
    int e = (int)hipGetLastError();
    if (e != 0)
        return e;
    const size_t lds = (size_t)T * sizeof(float) + ((size_t)k_top * sizeof(uint16_t) + 15) / 16 * 16;
    hipLaunchKernelGGL((k_topk_select<D, Meta>), dim3((unsigned)pairs), dim3(256), lds, st, c.v_codes,
                       meta<Meta>(c.v_min), meta<Meta>(c.v_scale), ws, static_cast<_Float16 *>(out), sel, c.S, T, k_top);
    return (int)hipGetLastError();
}

template <typename Meta>
int launch_quantize_m(const CachePlanes &c, const void *k, const void *v, int b, int s_src, int t_dst0,
                      hipStream_t st)
{
    switch (c.d) {
    case 64: return launch_quantize_d<64, Meta>(c, k, v, b, s_src, t_dst0, st);
    case 128: return launch_quantize_d<128, Meta>(c, k, v, b, s_src, t_dst0, st);
    default: return launch_quantize_d<256, Meta>(c, k, v, b, s_src, t_dst0, st);
    }
}

template <typename Meta>
int launch_decode_m(const CachePlanes &c, int pairs, const void *q, int T, void *out, const DecodeShape &sh,
                    float *ws, const void *k_new, const void *v_new, hipStream_t st)
{
    switch (c.d) {
    case 64: return launch_decode_d<64, Meta>(c, pairs, q, T, out, sh, ws, k_new, v_new, st);
    case 128: return launch_decode_d<128, Meta>(c, pairs, q, T, out, sh, ws, k_new, v_new, st);
    default: return launch_decode_d<256, Meta>(c, pairs, q, T, out, sh, ws, k_new, v_new, st);
    }
}

template <typename Meta>
int launch_topk_m(const CachePlanes &c, int pairs, const void *q, int T, int k_top, void *out, int32_t *sel,
                  float *ws, hipStream_t st)
{
    switch (c.d) {
    case 64: return launch_topk_d<64, Meta>(c, pairs, q, T, k_top, out, sel, ws, st);
    case 128: return launch_topk_d<128, Meta>(c, pairs, q, T, k_top, out, sel, ws, st);
    default: return launch_topk_d<256, Meta>(c, pairs, q, T, k_top, out, sel, ws, st);
    }
}

// Quantise a weight matrix W [N][K] (fp16, row-major): group gi = n*(K/64) + g
// of 64 contiguous k is read by 8 lanes, coded with the binary16-metadata
// codec, and stored in the tiled layout the projection kernel streams: tile
// (n/64, g/2) of 4 KB codes, row n%64 at byte 64*(n%64), half g%2 at byte 32;
// min and scale at tile*128 + 2*(n%64) + g%2.
__global__ __launch_bounds__(256) void k_quantize_w(const uint4 *__restrict__ w, int64_t groups, int gk,
                                                    uint32_t *__restrict__ codes, _Float16 *__restrict__ mins,
                                                    _Float16 *__restrict__ scales)
{
    constexpr int R = 4;
    const int lir = threadIdx.x & 7;
    const int64_t g0 = (int64_t)blockIdx.x * (32 * R) + (threadIdx.x >> 3);
    uint4 x[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int64_t gi = min(g0 + 32 * u, groups - 1);
        x[u] = ld_stream16(w + gi * 8 + lir);
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
        uint32_t word;
        float mn, sc;
        quant_lane8<_Float16>(x[u], word, mn, sc);
        const int64_t gi = g0 + 32 * u;
        if (gi < groups) {
            const int64_t n = gi / gk, g = gi - n * gk;
            const int64_t slot = ((n >> 6) * (gk >> 1) + (g >> 1)) * 128 + (n & 63) * 2 + (g & 1);
            __builtin_nontemporal_store(word, codes + slot * 8 + lir);
            if (lir == 0) {
                __builtin_nontemporal_store((_Float16)mn, mins + slot);
                __builtin_nontemporal_store((_Float16)sc, scales + slot);
            }
        }
    }
}

} // namespace

int launch_quantize_weight(const void *w, int N, int K, uint8_t *codes, void *mins, void *scales, hipStream_t st)
{
    const int64_t groups = (int64_t)N * (K / 64);
    const int64_t per_block = 32 * 4;
    hipLaunchKernelGGL(k_quantize_w, dim3((unsigned)((groups + per_block - 1) / per_block)), dim3(256), 0, st,
                       static_cast<const uint4 *>(w), groups, K / 64, reinterpret_cast<uint32_t *>(codes),
                       static_cast<_Float16 *>(mins), static_cast<_Float16 *>(scales));
    return (int)hipGetLastError();
}

int launch_quantize(const CachePlanes &c, const void *k, const void *v, int b, int s_src, int t_dst0,
                    hipStream_t st)
{
    return c.meta_f16 ? launch_quantize_m<_Float16>(c, k, v, b, s_src, t_dst0, st)
                      : launch_quantize_m<float>(c, k, v, b, s_src, t_dst0, st);
}

int launch_decode(const CachePlanes &c, int pairs, const void *q, int T, void *out, const DecodeShape &sh,
                  float *ws, const void *k_new, const void *v_new, hipStream_t st)
{
    return c.meta_f16 ? launch_decode_m<_Float16>(c, pairs, q, T, out, sh, ws, k_new, v_new, st)
                      : launch_decode_m<float>(c, pairs, q, T, out, sh, ws, k_new, v_new, st);
}

// Device address of `scratch` on the device `st` belongs to (the current
// device for the null stream), looked up once per device with that device
// current and kept for the life of the process.  Returns a hipError_t.
constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mu;
static float *g_scratch_ptr[kMaxScratchDevices] = {};

int noalloc_scratch(hipStream_t st, float **ptr)
{
    int dev = -1;
    hipError_t e = st != nullptr ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return (int)e;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return (int)e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return (int)e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess)
            return (int)e;
        if (e2 != hipSuccess)
            return (int)e2;
        if (p == nullptr)
            return (int)hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<float *>(p);
    }
    *ptr = g_scratch_ptr[dev];
    return 0;
}

int launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st)
{
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t blocks = (n16 + 256 * 16 - 1) / (256 * 16);
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const uint4 *>(buf), n16,
                       sink);
    return (int)hipGetLastError();
}

// The codec's scale and inverse for each given range (codec_params, the code
// path every quantiser takes).
template <typename Meta>
__global__ __launch_bounds__(256) void k_codec_params(const float *__restrict__ rng, int64_t n,
                                                      float *__restrict__ scale, float *__restrict__ inv)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        float s, v;
        codec_params<Meta>(rng[i], s, v);
        scale[i] = s;
        inv[i] = v;
    }
}

int launch_codec_params(const float *rng, int64_t n, bool meta_f16, float *scale, float *inv, hipStream_t st)
{
    const dim3 grid((unsigned)((n + 255) / 256));
    if (meta_f16)
        hipLaunchKernelGGL(k_codec_params<_Float16>, grid, dim3(256), 0, st, rng, n, scale, inv);
    else
        hipLaunchKernelGGL(k_codec_params<float>, grid, dim3(256), 0, st, rng, n, scale, inv);
    return (int)hipGetLastError();
}

size_t decode_ws_floats(int pairs, int d, int splits)
{
    return splits > 1 ? (size_t)splits * (size_t)pairs * (size_t)(d + 2) : 0;
}


size_t topk_ws_floats(int pairs, int T) { return (size_t)pairs * (size_t)T; }

int launch_topk(const CachePlanes &c, int pairs, const void *q, int T, int k_top, void *out, int32_t *sel,
                float *ws, hipStream_t st)
{
    return c.meta_f16 ? launch_topk_m<_Float16>(c, pairs, q, T, k_top, out, sel, ws, st)
                      : launch_topk_m<float>(c, pairs, q, T, k_top, out, sel, ws, st);
}

} // namespace kvq
