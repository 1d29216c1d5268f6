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
// The group codec for one lane's 8 consecutive fp16 values; 8 consecutive
// lanes (an aligned 8-lane group) hold one 64-element group.  Every lane of
// the wave must be active (DPP).  Binary32, one rounding per operation:
// min/max over the group (exact; -0 -> +0), rng = max - min, then
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
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = h2f_lo(w[j]);
        f[2 * j + 1] = h2f_hi(w[j]);
    }
    float mn = f[0], mx = f[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        mn = fminf(mn, f[i]);
        mx = fmaxf(mx, f[i]);
    }
    mn = fminf(mn, dpp<kQuadXor1>(mn));
    mx = fmaxf(mx, dpp<kQuadXor1>(mx));
    mn = fminf(mn, dpp<kQuadXor2>(mn));
    mx = fmaxf(mx, dpp<kQuadXor2>(mx));
    mn = fminf(mn, dpp<kHalfRowMirror>(mn));
    mx = fmaxf(mx, dpp<kHalfRowMirror>(mx));
    mn = mn + 0.0f; // -0 -> +0
    mx = mx + 0.0f;
    const float rng = mx - mn;
    uint32_t codes = 0;
    float scale = 0.0f, inv = 0.0f;
    if constexpr (sizeof(Meta) == 4) {
        if (rng != 0.0f) {
            scale = rng / 15.0f; // correctly rounded (HIP default division)
            inv = 15.0f / rng;
        }
    } else {
        if (rng != 0.0f)
            scale = (float)(_Float16)(rng / 15.0f); // binary16, nearest, ties to even
        if (scale != 0.0f)
            inv = 1.0f / scale;
    }
    if (scale != 0.0f) {
        // v_cvt_pk_u8_f32 rounds to nearest even, takes t <= 0 to 0 and inserts the
        // byte: the codes of the even elements go to bytes of ev, the odd ones to od,
        // and ev | od << 4 puts element i at bits 4i.  With binary32 metadata t never
        // reaches 15.5 (t <= 15 (1 + 2^-24)^2), so no clamp is needed; with binary16
        // metadata the stored scale can be below rng/15 and t is clamped at 15 first.
        uint32_t ev = 0, od = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float t = f[i] - mn;
            t = t * inv;
            if constexpr (sizeof(Meta) != 4)
                t = fminf(t, 15.0f);
            if (i % 2 == 0)
                ev = __builtin_amdgcn_cvt_pk_u8_f32(t, i / 2, ev);
            else
                od = __builtin_amdgcn_cvt_pk_u8_f32(t, i / 2, od);
        }
        codes = ev | (od << 4);
    }
    word = codes;
    mn_out = mn;
    scale_out = scale;
}

} // namespace
} // namespace kvq
