// HIP kernels for gfx950: the decode projections y = x W^T with group-wise
// int4 weights ("FlexGen研究学术报告" section 三.2(C): weights compressed with
// the same group-wise asymmetric 4-bit code as the KV cache, 64 contiguous
// elements per group, dequantised to FP16 before compute; the FlexGen blog's
// "解码阶段" projections t W_Q, t W_K, t W_V and t_out W_O).
//
// W is [N][K] (output row n, input column k), quantised in groups of 64
// contiguous k with binary16 min/scale.  On the device the planes are tiled
// so that what one wave consumes per step is contiguous: tile (nt, kt) holds
// rows 64nt..64nt+63 and k = 128kt..128kt+127, 4 KB of codes (row r at byte
// 64r, even k in the low nibble) and 128 mins / 128 scales (row r, group h at
// 2r+h).  The dequantised
// weight is the binary16 value nearest to min + c*scale, computed with one
// packed fp16 FMA (exact product and sum, one rounding), and the product runs
// on the matrix cores: v_mfma_f32_16x16x32_f16, binary32 accumulation.
//
// Shape of the work (OPT-175B decode: M = 144 tokens, N = K = 12288): the
// weight stream (N*K/2 bytes) and the matrix-core time are of the same order,
// so the kernel keeps both busy: a workgroup owns a 16*MB x 256 output tile
// (MB <= 9 row blocks of 16) and a range of K; its eight waves (two per SIMD)
// each take 32 columns and all the row blocks, share each 128-wide chunk of x
// through LDS (double-buffered), and stream and dequantise their own 32
// weight rows.  Ranges of K are split across
// workgroups when the column tiles alone cannot fill the 256 CUs; the split
// partials (binary32) are summed by a second kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq4_launch.h"

namespace kvq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 128;          // k per pipeline step
constexpr int kPitch = kChunk + 8;   // LDS row pitch of the x chunk, halves (breaks bank aliasing)
constexpr int kColsPerWave = 64;     // four 16-column blocks
constexpr int kColsPerGroup = 4 * kColsPerWave;
constexpr int kThreads = 512;        // 8 waves
// Work of a wave: kGemmWaveColBlocks = 4: 64 columns and half of the row
// blocks (8 waves = 4 column groups x 2 row halves); 2: 32 columns and all
// the row blocks (8 waves side by side), each weight dequantised once.
#ifndef KVQ_GEMM_WAVE_COL_BLOCKS
#define KVQ_GEMM_WAVE_COL_BLOCKS 2
#endif
constexpr int kGemmWaveColBlocks = KVQ_GEMM_WAVE_COL_BLOCKS;

__device__ __forceinline__ uint4 ld_nt16(const void *p)
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Reorder the 8 halves of a 16-byte x piece to (x0,x4,x1,x5,x2,x6,x3,x7): the
// order in which the weight unpack below yields its pairs.  The contraction
// index may be permuted freely as long as both operands agree.
__device__ __forceinline__ uint4 interleave_halves(uint4 v)
{
    // v.x=(x0,x1) v.y=(x2,x3) v.z=(x4,x5) v.w=(x6,x7)
    uint4 r;
    r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u); // (x0, x4)
    r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u); // (x1, x5)
    r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u); // (x2, x6)
    r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u); // (x3, x7)
    return r;
}

// The 8 codes of a dword (k = k0..k0+7) as dequantised binary16 weights in
// the order (w0,w4),(w1,w5),(w2,w6),(w3,w7).  Each code is made exact in
// binary16 (OR-ing the pattern of 1024 onto a nibble at bits 0..3 gives 1024+c,
// OR-ing 64 onto bits 4..7 gives 64+c; subtracting the bias is exact), then
// one packed FMA forms min + c*scale with a single rounding.  The OR
// constants sit in VGPRs (magic) so each pair is one v_and_or_b32: GFX9's
// VOP3 takes no literal operand.
struct Magic16 {
    uint32_t m1024, m64;
};
__device__ __forceinline__ Magic16 magic16()
{
    Magic16 m;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m.m1024));
    asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(m.m64));
    return m;
}

__device__ __forceinline__ h8 dequant8(uint32_t w, h2 sc, h2 mn, const Magic16 mg)
{
    const uint32_t y = w >> 8;
    const h2 b1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
    const h2 b64 = {(_Float16)-64.0f, (_Float16)-64.0f};
    const h2 c0 = __builtin_bit_cast(h2, (w & 0x000F000Fu) | mg.m1024) + b1024;
    const h2 c1 = __builtin_bit_cast(h2, (w & 0x00F000F0u) | mg.m64) + b64;
    const h2 c2 = __builtin_bit_cast(h2, (y & 0x000F000Fu) | mg.m1024) + b1024;
    const h2 c3 = __builtin_bit_cast(h2, (y & 0x00F000F0u) | mg.m64) + b64;
    const uint4 d = make_uint4(__builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c0, sc, mn)),
                               __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c1, sc, mn)),
                               __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c2, sc, mn)),
                               __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c3, sc, mn)));
    return __builtin_bit_cast(h8, d);
}

// One wave's weights for one 128-k chunk: for each of its CB column blocks of
// 16, lane l holds column (block*16 + l%16), k = 32*(l/16) .. +31 of the chunk
// (16 code bytes) and that range's group min and scale.
template <int CB>
struct WChunk {
    uint4 code[CB];
    uint32_t mn[CB], sc[CB]; // binary16 bits, low half
};

// Element at a 32-bit byte offset from a wave-uniform base (the load then
// takes the scalar-base + 32-bit-offset form).
template <typename T>
__device__ __forceinline__ const T *at_byte(const T *base, uint32_t off)
{
    return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + off);
}

// Chunk c of the wave's 16*CB rows starting at n0 (n0 % 64 + 16*CB <= 64):
// part of one 4 KB tile, lane l reading 16 bytes of row n0%64 + 16b + l%16 at
// byte 16*(l/16).
template <int CB>
__device__ __forceinline__ WChunk<CB> load_w_chunk(const uint8_t *__restrict__ codes,
                                                   const uint16_t *__restrict__ mins,
                                                   const uint16_t *__restrict__ scales, int64_t n0, int K, int c,
                                                   int lane)
{
    const int64_t tile = (n0 >> 6) * (K / kChunk) + c; // wave-uniform
    const uint8_t *ct = codes + tile * 4096;
    const uint16_t *mt = mins + tile * 128, *st = scales + tile * 128;
    WChunk<CB> w;
#pragma unroll
    for (int b = 0; b < CB; ++b) {
        const uint32_t r = (uint32_t)(n0 & 63) + b * 16 + (lane & 15);
        w.code[b] = ld_nt16(ct + (r * 64 + 16 * (lane >> 4)));
        w.mn[b] = __builtin_nontemporal_load(at_byte(mt, 4 * r + 2 * (lane >> 5)));
        w.sc[b] = __builtin_nontemporal_load(at_byte(st, 4 * r + 2 * (lane >> 5)));
    }
    return w;
}

// Rows m0 .. m0+16*MB-1 of x[:, kc .. kc+127], in 16*MB*16 pieces of 8
// halves; thread t holds pieces t, t+512, ...  Loaded into registers first
// and written to LDS later, so the loads are in flight during the matrix work.
template <int MB>
struct XStage {
    static constexpr int PIECES = 16 * MB * (kChunk / 8);
    static constexpr int PER_THREAD = (PIECES + kThreads - 1) / kThreads;
    uint4 v[PER_THREAD];
};

// Per-thread byte offsets of its pieces' rows (fixed over the K loop; rows
// past M, and pieces past the tile, point at row M-1 and are zeroed), and
// whether the tile has such rows at all.
template <int MB>
struct XOffsets {
    uint32_t off[XStage<MB>::PER_THREAD];
    uint32_t ok; // bit i: piece i is a real row
    bool partial;
};

template <int MB>
__device__ __forceinline__ XOffsets<MB> x_offsets(int M, int K, int m0)
{
    XOffsets<MB> o;
    o.ok = 0;
#pragma unroll
    for (int i = 0; i < XStage<MB>::PER_THREAD; ++i) {
        const int p = threadIdx.x + kThreads * i;
        const int row = (p >> 4) % (16 * MB), kp = p & 15;
        const int rc = min(m0 + row, M - 1);
        o.off[i] = (uint32_t)(((int64_t)rc * K + 8 * kp) * 2);
        if (p < XStage<MB>::PIECES && m0 + row < M)
            o.ok |= 1u << i;
    }
    o.partial = m0 + 16 * MB > M || XStage<MB>::PIECES % kThreads != 0;
    return o;
}

// x of chunk kc: a uniform base plus the per-thread offsets (M*K*2 < 2^32).
template <int MB>
__device__ __forceinline__ void load_x(const uint16_t *__restrict__ x, int kc, const XOffsets<MB> &o,
                                       XStage<MB> &xs)
{
    const uint16_t *xb = x + kc;
#pragma unroll
    for (int i = 0; i < XStage<MB>::PER_THREAD; ++i)
        xs.v[i] = ld_nt16(at_byte(xb, o.off[i]));
    if (o.partial) { // uniform
#pragma unroll
        for (int i = 0; i < XStage<MB>::PER_THREAD; ++i)
            if (!((o.ok >> i) & 1u))
                xs.v[i] = make_uint4(0, 0, 0, 0);
    }
}

// Write a staged chunk to LDS (rows >= M are zero), each piece reordered by
// interleave_halves.
template <int MB>
__device__ __forceinline__ void store_x(const XStage<MB> &xs, _Float16 *__restrict__ sx)
{
#pragma unroll
    for (int i = 0; i < XStage<MB>::PER_THREAD; ++i) {
        const int p = threadIdx.x + kThreads * i;
        if (p < XStage<MB>::PIECES)
            *reinterpret_cast<uint4 *>(sx + (p >> 4) * kPitch + 8 * (p & 15)) = interleave_halves(xs.v[i]);
    }
}

// One 128-k chunk of one wave: dequantise its weights k-step by k-step and
// accumulate its MBW x CB blocks (row blocks rb0 .. rb0+MBW-1 of the x chunk
// in LDS).
template <int MBW, int CB>
__device__ __forceinline__ void mma_chunk(const WChunk<CB> &cur, const _Float16 *__restrict__ sxb, int rb0, int lane,
                                          f4 (&acc)[MBW > 0 ? MBW : 1][CB])
{
    if constexpr (MBW > 0) {
        const Magic16 mg = magic16();
        h2 sc[CB], mn[CB];
#pragma unroll
        for (int b = 0; b < CB; ++b) {
            sc[b] = __builtin_bit_cast(h2, (cur.sc[b] & 0xFFFFu) * 0x00010001u);
            mn[b] = __builtin_bit_cast(h2, (cur.mn[b] & 0xFFFFu) * 0x00010001u);
        }
        auto word = [&](int b, int j) -> uint32_t {
            return j == 0 ? cur.code[b].x : j == 1 ? cur.code[b].y : j == 2 ? cur.code[b].z : cur.code[b].w;
        };
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h8 bw[CB];
#pragma unroll
            for (int b = 0; b < CB; ++b)
                bw[b] = dequant8(word(b, j), sc[b], mn[b], mg);
            // all of this k-step's x reads are issued before its products
            h8 a[MBW];
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
                a[mb] = *reinterpret_cast<const h8 *>(sxb + ((rb0 + mb) * 16 + (lane & 15)) * kPitch +
                                                      32 * (lane >> 4) + 8 * j);
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
                for (int b = 0; b < CB; ++b)
                    acc[mb][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mb], bw[b], acc[mb][b], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, MBW, 0);      // the k-step's LDS reads,
            __builtin_amdgcn_sched_group_barrier(0x008, CB * MBW, 0); // then its products
        }
    }
    // keep the caller's LDS writes of the next x chunk (and their wait on its
    // global loads) after this chunk's products
    __builtin_amdgcn_sched_barrier(0);
}

// The K loop and the stores of one wave: its 16*CB columns starting at n0 and
// its MBW row blocks starting at block rb0 of the tile (the tile's MB blocks
// are staged in LDS by all waves).  Every wave runs the same sequence of
// barriers whatever its MBW.
template <int MB, int MBW, int CB>
__device__ __forceinline__ void gemm_wave(const uint16_t *__restrict__ x, const uint8_t *__restrict__ codes,
                                          const uint16_t *__restrict__ mins, const uint16_t *__restrict__ scales,
                                          _Float16 *__restrict__ y, float *__restrict__ ws, int M, int N, int K,
                                          int m0, int64_t n0, int rb0, int split, int splits, int c_begin, int c_end,
                                          _Float16 (*sx)[16 * MB * kPitch])
{
    const int lane = threadIdx.x & 63;
    const bool wave_ok = n0 < N; // N % 64 == 0: a wave's columns are all in range or all out
    const int64_t nsafe = wave_ok ? n0 : 0; // waves past N stream rows 0.. and store nothing
    f4 acc[MBW > 0 ? MBW : 1][CB];
#pragma unroll
    for (int mb = 0; mb < (MBW > 0 ? MBW : 1); ++mb)
#pragma unroll
        for (int b = 0; b < CB; ++b)
            acc[mb][b] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    XStage<MB> xs;
    const XOffsets<MB> xo = x_offsets<MB>(M, K, m0);
    WChunk<CB> cur{};
    if (c_begin < c_end) {
        if constexpr (MBW > 0)
            cur = load_w_chunk<CB>(codes, mins, scales, nsafe, K, c_begin, lane);
        load_x<MB>(x, c_begin * kChunk, xo, xs);
        store_x<MB>(xs, sx[0]);
    }
    __syncthreads();
    for (int c = c_begin; c < c_end; ++c) {
        const int buf = (c - c_begin) & 1;
        const bool more = c + 1 < c_end; // uniform
        WChunk<CB> nxt{};
        if (more) {
            if constexpr (MBW > 0)
                nxt = load_w_chunk<CB>(codes, mins, scales, nsafe, K, c + 1, lane);
            load_x<MB>(x, (c + 1) * kChunk, xo, xs);
        }
        mma_chunk<MBW, CB>(cur, sx[buf], rb0, lane, acc);
        if (more)
            store_x<MB>(xs, sx[buf ^ 1]);
        cur = nxt;
        __syncthreads();
    }

    if constexpr (MBW > 0) {
        if (!wave_ok)
            return;
        // D layout: lane l holds rows 4*(l/16) .. +3 of column l%16 of each 16x16 block
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
#pragma unroll
            for (int b = 0; b < CB; ++b) {
                const int64_t n = n0 + b * 16 + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + (rb0 + mb) * 16 + 4 * (lane >> 4) + r;
                    if (m < M) {
                        if (splits == 1)
                            y[(int64_t)m * N + n] = (_Float16)acc[mb][b][r];
                        else
                            ws[((int64_t)split * M + m) * N + n] = acc[mb][b][r];
                    }
                }
            }
        }
    }
}

// grid.x: column groups of 256 (fastest), grid.y: K splits, grid.z: row tiles
// of 16*MB.  Eight waves, two per SIMD, so one's dequantisation overlaps the
// other's matrix work.  CB = 2 (the default): wave w takes columns 32w of the
// group and all MB row blocks, so every weight is dequantised once.  CB = 4:
// wave w takes columns 64*(w%4) and the upper (w < 4: ceil(MB/2) blocks) or
// lower (w >= 4) row blocks; the two waves of a column group stream and
// dequantise the same weight tile.  Measured on the OPT-175B projections, CB = 2
// against CB = 4: QKV at M = 144, 64, 32: 251.7 -> 229.7, 157.4 -> 104.9,
// 123.7 -> 82.3 us; output at M = 64, 32: 59.8 -> 48.3, 58.0 -> 42.6 us
// (bit-identical results).
// splits == 1: y written as fp16; else binary32 partials to ws[split][M][N].
// The next chunk's weights and x are loaded into registers while the current
// chunk is multiplied; x then goes to the other LDS buffer.
template <int MB, int CB>
__global__ __launch_bounds__(kThreads) void k_gemm_w4(const uint16_t *__restrict__ x,
                                                      const uint8_t *__restrict__ codes,
                                                      const uint16_t *__restrict__ mins,
                                                      const uint16_t *__restrict__ scales,
                                                      _Float16 *__restrict__ y, float *__restrict__ ws, int M,
                                                      int N, int K, int chunks_per_split)
{
    constexpr int MH = (MB + 1) / 2;
    __shared__ __attribute__((aligned(16))) _Float16 sx[2][16 * MB * kPitch];
    const int wave = threadIdx.x >> 6;
    const int split = blockIdx.y, splits = gridDim.y;
    const int m0 = blockIdx.z * 16 * MB;
    const int c_begin = split * chunks_per_split;
    const int c_end = min(K / kChunk, c_begin + chunks_per_split);
    if constexpr (CB == 4) {
        const int64_t n0 = (int64_t)blockIdx.x * kColsPerGroup + (wave & 3) * kColsPerWave;
        if (wave < 4)
            gemm_wave<MB, MH, 4>(x, codes, mins, scales, y, ws, M, N, K, m0, n0, 0, split, splits, c_begin, c_end,
                                 sx);
        else
            gemm_wave<MB, MB - MH, 4>(x, codes, mins, scales, y, ws, M, N, K, m0, n0, MH, split, splits, c_begin,
                                      c_end, sx);
    } else {
        const int64_t n0 = (int64_t)blockIdx.x * kColsPerGroup + wave * 16 * CB;
        gemm_wave<MB, MB, CB>(x, codes, mins, scales, y, ws, M, N, K, m0, n0, 0, split, splits, c_begin, c_end, sx);
    }
}

// y[m][n] = fp16(sum over splits of ws[s][m][n]), 4 outputs per thread.
__global__ __launch_bounds__(256) void k_gemm_reduce(const float *__restrict__ ws, _Float16 *__restrict__ y,
                                                     int64_t mn, int splits)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= mn)
        return;
    float4 s = *reinterpret_cast<const float4 *>(ws + i);
    for (int k = 1; k < splits; ++k) {
        const float4 t = *reinterpret_cast<const float4 *>(ws + (int64_t)k * mn + i);
        s.x += t.x;
        s.y += t.y;
        s.z += t.z;
        s.w += t.w;
    }
    y[i] = (_Float16)s.x;
    y[i + 1] = (_Float16)s.y;
    y[i + 2] = (_Float16)s.z;
    y[i + 3] = (_Float16)s.w;
}

template <int MB>
int launch_gemm_mb(const GemmArgs &g, hipStream_t st)
{
    const dim3 grid((unsigned)((g.N + kColsPerGroup - 1) / kColsPerGroup), (unsigned)g.splits,
                    (unsigned)((g.M + 16 * MB - 1) / (16 * MB)));
    hipLaunchKernelGGL((k_gemm_w4<MB, kGemmWaveColBlocks>), grid, dim3(kThreads), 0, st, static_cast<const uint16_t *>(g.x), g.codes,
                       static_cast<const uint16_t *>(g.mins), static_cast<const uint16_t *>(g.scales),
                       static_cast<_Float16 *>(g.y), g.ws, g.M, g.N, g.K, g.chunks_per_split);
    int e = (int)hipGetLastError();
    if (e != 0 || g.splits == 1)
        return e;
    const int64_t mn = (int64_t)g.M * g.N; // N % 64 == 0, so mn % 4 == 0
    hipLaunchKernelGGL(k_gemm_reduce, dim3((unsigned)((mn / 4 + 255) / 256)), dim3(256), 0, st, g.ws,
                       static_cast<_Float16 *>(g.y), mn, g.splits);
    return (int)hipGetLastError();
}

} // namespace

int gemm_row_blocks(int M) { return M >= 144 ? 9 : (M + 15) / 16; }

int launch_gemm_w4(const GemmArgs &g, hipStream_t st)
{
    switch (gemm_row_blocks(g.M)) {
    case 1: return launch_gemm_mb<1>(g, st);
    case 2: return launch_gemm_mb<2>(g, st);
    case 3: return launch_gemm_mb<3>(g, st);
    case 4: return launch_gemm_mb<4>(g, st);
    case 5: return launch_gemm_mb<5>(g, st);
    case 6: return launch_gemm_mb<6>(g, st);
    case 7: return launch_gemm_mb<7>(g, st);
    case 8: return launch_gemm_mb<8>(g, st);
    default: return launch_gemm_mb<9>(g, st);
    }
}

} // namespace kvq
