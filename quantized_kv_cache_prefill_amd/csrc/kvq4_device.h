// Device helpers shared by the HIP kernels of this library: DPP lane
// exchange, fp16 widening, streaming loads and the group codec.
//
// The codec follows "FlexGen研究学术报告" section 三.2(C): group-wise
// asymmetric 4-bit quantisation, 64 contiguous elements per group (group axis
// = head_dim, min/max affine code with scale (max-min)/15 and round-half-even
// codes; binary32 or binary16 min/scale).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// DPP controls (GFX9 encoding).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kHalfRowMirror = 0x141; // lane i <-> lane 7-i inside each 8-lane group

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF,
                                                                 false));
}

__device__ __forceinline__ float h2f_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float h2f_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// Loads of data that is used exactly once (the cache planes, the prompt
// K/V): nontemporal, so they stream through without displacing other lines.
// On MI355X this raises a plain 16-byte streaming read from ~6.3 to ~7.0 TB/s.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void *p)
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float ld_stream(const float *p) { return __builtin_nontemporal_load(p); }
// ===========================================================================
// The group codec's two divisions, exact in binary32 for every range the codec
// can meet (rng a positive binary32 value up to 2 x 65504; 0 is handled by the
// caller), without the generic division sequence (scaling, fix-up):
//  * scale = rng/15: q0 = rng * c with c = the binary32 value nearest 1/15,
//    then one correction with the exact residual rng - 15 q0 (a fused
//    multiply-add), the scheme for division by a constant known in advance;
//  * inv = 15/rng: the hardware reciprocal (within 1 ulp), one Newton step,
//    q = 15 y, then the same residual correction;
//  * binary16 metadata: scale = rng/15 as above, rounded to binary16 (nearest,
//    ties to even), and inv = 1/scale by reciprocal + Newton + residual
//    correction.
// Every result is the correctly rounded quotient; this is checked for every
// binary32 range in [2^-24, 2^17] through kvq_codec_params.  scale_out and
// inv_out are 0 when the stored scale is 0.
// ===========================================================================
template <typename Meta>
__device__ __forceinline__ void codec_params(float rng, float &scale_out, float &inv_out)
{
#pragma clang fp contract(off)
    constexpr float c15 = 1.0f / 15.0f;
    const float q0 = rng * c15;
    float scale = __builtin_fmaf(__builtin_fmaf(-q0, 15.0f, rng), c15, q0);
    float den = rng, num = 15.0f;
    if constexpr (sizeof(Meta) != 4) {
        // binary16, nearest, ties to even, of the binary32 quotient: the empty asm
        // keeps the compiler from rounding the fused multiply-add straight to
        // binary16 (one rounding instead of the two the codec defines).
        asm("" : "+v"(scale));
        scale = (float)(_Float16)scale;
        den = scale;
        num = 1.0f;
    }
    float y = __builtin_amdgcn_rcpf(den);
    y = __builtin_fmaf(__builtin_fmaf(-den, y, 1.0f), y, y);
    const float q = num * y;
    const float inv = __builtin_fmaf(__builtin_fmaf(-q, den, num), y, q);
    scale_out = scale;
    inv_out = scale != 0.0f ? inv : 0.0f;
}

// Packed binary16 min / max (IEEE minNum / maxNum per half).  Written out so
// that the compiler adds no NaN-quieting step before each use: the codec's
// inputs are finite.
__device__ __forceinline__ uint32_t pk_min16(uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ uint32_t pk_max16(uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// (a.lo, b.lo) and (a.hi, b.hi) -> (min(a.lo, a.hi), min(-b.lo, -b.hi)).
__device__ __forceinline__ uint32_t pk_min_neg_hi(uint32_t a, uint32_t b)
{
    const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x05040100u); // (a.lo, b.lo)
    const uint32_t hi = __builtin_amdgcn_perm(b, a, 0x07060302u); // (a.hi, b.hi)
    uint32_t r;
    asm("v_pk_min_f16 %0, %1, %2 neg_lo:[0,0] neg_hi:[1,1]" : "=v"(r) : "v"(lo), "v"(hi));
    return r;
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// x - m in binary32 (one rounding) for the low / high binary16 half of w,
// widened inside the fused multiply-add (x * 1 - m).
__device__ __forceinline__ float sub_lo16(uint32_t w, float m)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(m));
    return r;
}
__device__ __forceinline__ float sub_hi16(uint32_t w, float m)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(m));
    return r;
}

// ===========================================================================
// The group codec for one lane's 8 consecutive fp16 values; 8 consecutive
// lanes (an aligned 8-lane group) hold one 64-element group.  Every lane of
// the wave must be active (DPP).  Binary32, one rounding per operation:
// min/max over the group (exact: taken on the binary16 values, -0 -> +0),
// rng = max - min, then
//  * binary32 metadata (Meta = float): scale = rng/15, inv = 15/rng (correctly
//    rounded divisions);
//  * binary16 metadata (Meta = _Float16): scale = rng/15 rounded to the nearest
//    binary16 value (ties to even), inv = 1/scale, so the codes are taken
//    against the stored scale; the min is an fp16 input, stored exactly;
// code = clamp(rint_even((x - min) * inv), 0, 15); a stored scale of 0
// (constant group, or a binary16 scale that underflows) gives codes 0.
// Inputs are finite fp16 values (the caller's contract).
// word holds the lane's 8 codes, element i at bits 4i..4i+3; mn_out and
// scale_out are the stored values, widened to binary32.
// ===========================================================================
template <typename Meta>
__device__ __forceinline__ void quant_lane8(const uint4 x, uint32_t &word, float &mn_out, float &scale_out)
{
#pragma clang fp contract(off)
    // Lane min and max of the 8 values, packed as (min, -max) so that each of
    // the three cross-lane steps is one exchange and one packed min.
    const uint32_t lo = pk_min16(pk_min16(x.x, x.y), pk_min16(x.z, x.w));
    const uint32_t hi = pk_max16(pk_max16(x.x, x.y), pk_max16(x.z, x.w));
    uint32_t p = pk_min_neg_hi(lo, hi);
    p = pk_min16(p, dpp_u<kQuadXor1>(p));
    p = pk_min16(p, dpp_u<kQuadXor2>(p));
    p = pk_min16(p, dpp_u<kHalfRowMirror>(p));
    const float mn = h2f_lo(p) + 0.0f; // -0 -> +0
    const float mx = -h2f_hi(p) + 0.0f;
    const float rng = mx - mn;
    float scale, inv;
    codec_params<Meta>(rng, scale, inv);
    // v_cvt_pk_u8_f32 rounds to nearest even, takes t <= 0 to 0 and inserts the
    // byte: the codes of the even elements go to bytes of ev, the odd ones to od,
    // and ev | od << 4 puts element i at bits 4i.  With binary32 metadata t never
    // reaches 15.5 (t <= 15 (1 + 2^-24)^2), so no clamp is needed; with binary16
    // metadata the stored scale can be below rng/15 and t is clamped at 15 first.
    // inv = 0 (scale 0) gives t = 0, code 0.
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
    word = ev | (od << 4);
    mn_out = mn;
    scale_out = scale;
}

} // namespace
} // namespace kvq
