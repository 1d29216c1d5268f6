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
// 2r+h).  The dequantised weight is the binary16 value nearest to
// min + c*scale, computed with one packed fp16 FMA (exact product and sum,
// one rounding), and the product runs on the matrix cores:
// v_mfma_f32_32x32x16_f16, binary32 accumulation.  On MI355X that
// instruction issues back to back at its full rate (32 cycles, 32768 flops);
// the 16x16x32 form measured 25.4 cycles per 16384 flops, 54% of the peak, so
// the rows of x are padded to a multiple of 32 instead.
//
// Shape of the work (OPT-175B decode: M = 144 tokens, N = K = 12288): the
// weight stream (N*K/2 bytes) and the matrix-core time are of the same order.
// A workgroup owns a 32*RB x 256 output tile (RB <= 5 row blocks of 32) and a
// range of K; its eight waves (two per SIMD, so that one hides the other's
// waits) each take 32 columns and all the row blocks.  x goes from HBM
// straight into LDS (buffer loads to LDS, 16-byte pieces XOR-swizzled within
// each row so the operand reads hit distinct banks) through a ring of three
// chunk buffers, two chunks ahead; each wave streams its own 32 weight rows
// through a ring of registers three chunks ahead and dequantises them as it
// multiplies, the operands of k-step s+1 fetched and dequantised between the
// products of step s.  Ranges of K are
// split across workgroups when the column tiles alone cannot fill the 256
// CUs; the split partials (binary32) are summed by a second kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq4_launch.h"

namespace kvq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int kChunk = 128;           // k per pipeline step
constexpr int kRowBytes = kChunk * 2; // bytes of one x row of a chunk (16 pieces of 16 bytes)
constexpr int kCB = 1;                // 32-column blocks per wave
constexpr int kColsPerWave = 32 * kCB;
constexpr int kWaves = 8;             // two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kColsPerGroup = kWaves * kColsPerWave;
constexpr int kDepth = 3;             // weight chunks in flight per wave (register ring)
constexpr int kXBuf = 3;              // x chunk buffers in LDS (x runs kXBuf - 1 chunks ahead)
constexpr int kWLoads = 4 * kCB;      // loads per weight chunk per lane (2 x 16 B codes, 2 x 2 B min/scale per block)
constexpr int kGroupsPerCU = 1;       // workgroups resident per CU (LDS: the x ring)
static_assert(kDepth == kXBuf, "the K loop is unrolled by one ring length for both rings");

// Buffer resources: a base, a size in bytes (loads at or past it return zeros
// and touch no memory) and the raw-buffer flags.  The K loop issues every load
// unconditionally -- a chunk past the range, and rows past M, get offsets
// beyond the size -- so the loads keep one fixed order.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr int kNT = 2;                     // cache policy: nontemporal (the weights are used once)
constexpr uint32_t kOutside = 0xFFFFFFC0u; // an offset past any resource (+ up to 63 still past it)
__device__ __forceinline__ uint4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT));
}
__device__ __forceinline__ uint32_t bld2(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kNT);
}
typedef __attribute__((address_space(3))) void lds_void_t;
// 16 bytes per lane, HBM -> LDS: lane l's bytes land at dst + 16 l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void *dst, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, (int)voff, 0, 0, 0);
}

// The 8 codes of a dword (k = k0..k0+7, code i at bits 4i..4i+3) as
// dequantised binary16 weights, in k order.  Each pair (e_2i, e_2i+1) is made
// exact in binary16: one byte permute puts byte i of the dword at bytes 0 and
// 2, the mask keeps e_2i at bits 0..3 and e_2i+1 at bits 20..23, OR-ing the
// patterns of 1024 and 64 onto them gives (1024 + e_2i, 64 + e_2i+1), and
// subtracting (1024, 64) is exact.  One packed FMA then forms min + c*scale
// with a single rounding.  `magic` sits in a VGPR: GFX9's VOP3 takes no
// literal operand and at most one scalar one.
__device__ __forceinline__ uint32_t magic_vgpr()
{
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x54006400" : "=v"(m));
    return m;
}

__device__ __forceinline__ h8 dequant8(uint32_t w, h2 sc, h2 mn, uint32_t magic)
{
    const h2 bias = {(_Float16)-1024.0f, (_Float16)-64.0f};
    constexpr uint32_t sel[4] = {0x0C000C00u, 0x0C010C01u, 0x0C020C02u, 0x0C030C03u};
    uint32_t d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = __builtin_amdgcn_perm(0u, w, sel[i]);
        const h2 c = __builtin_bit_cast(h2, (t & 0x00F0000Fu) | magic) + bias;
        d[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c, sc, mn));
    }
    return __builtin_bit_cast(h8, make_uint4(d[0], d[1], d[2], d[3]));
}

// One wave's weights for one 128-k chunk: for each of its kCB 32-column
// blocks, lane l holds column l%32 of the block and k = 64*(l/32) .. +63 of
// the chunk (32 code bytes, exactly one group) with that group's min and
// scale.  In k-step s (0..7) the lane's 8 operand values are k = 64*(l/32) +
// 8s .. +7: the two lane halves give the 16 k of the 32x32x16 product.
struct WChunk {
    uint4 code[kCB][2];
    uint32_t mn[kCB], sc[kCB]; // binary16 bits, low half
};

// The weight planes of one wave's 32 rows (half a row of 64-row tiles of the
// tiled layout: K/128 tiles of 4 KB codes and 128 mins / 128 scales each).
struct WStreams {
    __amdgpu_buffer_rsrc_t codes, mins, scales;
    uint32_t code_off, meta_off; // the lane's offsets inside a tile
};

__device__ __forceinline__ WStreams w_streams(const uint8_t *codes, const uint16_t *mins, const uint16_t *scales,
                                              int64_t n0, int K, int lane)
{
    const int64_t tiles = K / kChunk;
    const int64_t t0 = (n0 >> 6) * tiles; // wave-uniform
    WStreams w;
    w.codes = rsrc(codes + t0 * 4096, (uint32_t)(tiles * 4096));
    w.mins = rsrc(mins + t0 * 128, (uint32_t)(tiles * 256));
    w.scales = rsrc(scales + t0 * 128, (uint32_t)(tiles * 256));
    const uint32_t blk = (uint32_t)((n0 & 63) >> 5); // the wave's first 32-row block inside the tile
    w.code_off = blk * 2048u + (uint32_t)((lane & 31) * 64 + 32 * (lane >> 5));
    w.meta_off = blk * 128u + (uint32_t)(4 * (lane & 31) + 2 * (lane >> 5));
    return w;
}

// Chunk c of the wave's rows (an invalid chunk reads zeros): lane l reads 32
// bytes of row 32b + l%32 at byte 32*(l/32), and that group's min and scale.
__device__ __forceinline__ WChunk load_w_chunk(const WStreams &ws, uint32_t c, bool valid)
{
    WChunk w;
#pragma unroll
    for (int b = 0; b < kCB; ++b) {
        const uint32_t co = valid ? c * 4096u + (uint32_t)b * 2048u + ws.code_off : kOutside;
        const uint32_t mo = valid ? c * 256u + (uint32_t)b * 128u + ws.meta_off : kOutside;
        w.code[b][0] = bld16(ws.codes, co);
        w.code[b][1] = bld16(ws.codes, co + 16);
        w.mn[b] = bld2(ws.mins, mo);
        w.sc[b] = bld2(ws.scales, mo);
    }
    return w;
}

// x rows m0 .. m0+32*RB-1 of one chunk in LDS: row r at byte 256 r, its
// 16-byte piece j at slot j ^ (r & 15).  Thread t's u-th load fills 16-byte
// position p = 64 * (4u + wave) + lane, i.e. row p/16, slot p%16; off[u]
// holds the byte offset in x of the piece that belongs there (chunk 0), or
// kOutside for a row past M.
template <int RB>
struct XLoads {
    static constexpr int PER_THREAD = 32 * RB * 16 / kThreads; // 16 RB pieces per wave-row of lanes
    uint32_t off[PER_THREAD];
};

template <int RB>
__device__ __forceinline__ XLoads<RB> x_loads(int M, int K, int m0, int wave, int lane)
{
    XLoads<RB> o;
#pragma unroll
    for (int u = 0; u < XLoads<RB>::PER_THREAD; ++u) {
        const int p = 64 * (kWaves * u + wave) + lane;
        const int row = p >> 4, slot = p & 15;
        const int piece = slot ^ (row & 15);
        o.off[u] = m0 + row < M ? (uint32_t)(((int64_t)(m0 + row) * K + 8 * piece) * 2) : kOutside;
    }
    return o;
}

// Chunk c of x into the LDS buffer `dst` (an invalid chunk, and rows past M,
// read zeros).
template <int RB>
__device__ __forceinline__ void issue_x(__amdgpu_buffer_rsrc_t rx, const XLoads<RB> &o, uint32_t c, bool valid,
                                        char *dst, int wave)
{
#pragma unroll
    for (int u = 0; u < XLoads<RB>::PER_THREAD; ++u)
        dma16(rx, dst + 1024 * (kWaves * u + wave), valid && o.off[u] != kOutside ? o.off[u] + c * kRowBytes : kOutside);
}

// One 128-k chunk of one wave: eight k-steps, each multiplying the step's 8
// dequantised weights of both column blocks with the RB row blocks of the x
// chunk (lane l reads row 32rb + l%32, piece 8*(l/32) + s).  The x operands
// and the weights of step s+1 are read and dequantised before the products
// of step s are issued, and the scheduler spreads them between those
// products, so their latency and vector work overlap the matrix core.
template <int RB>
__device__ __forceinline__ void mma_chunk(const WChunk &cur, const char *__restrict__ sxb, int lane,
                                          f16v (&acc)[RB][kCB])
{
    const uint32_t magic = magic_vgpr();
    h2 sc[kCB], mn[kCB];
#pragma unroll
    for (int b = 0; b < kCB; ++b) {
        sc[b] = __builtin_bit_cast(h2, (cur.sc[b] & 0xFFFFu) * 0x00010001u);
        mn[b] = __builtin_bit_cast(h2, (cur.mn[b] & 0xFFFFu) * 0x00010001u);
    }
    auto word = [&](int b, int s) -> uint32_t {
        const uint4 q = cur.code[b][s >> 2];
        const int j = s & 3;
        return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
    };
    const int r = lane & 31, h = lane >> 5;
    const char *xrow = sxb + r * kRowBytes;
    auto ld_a = [&](int s, h8 (&a)[RB]) {
        const int slot = (8 * h + s) ^ (r & 15);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            a[rb] = *reinterpret_cast<const h8 *>(xrow + rb * 32 * kRowBytes + 16 * slot);
    };
    // x operands two k-steps ahead (a ring of three), weights one step ahead
    h8 a[3][RB], bw[2][kCB];
    ld_a(0, a[0]);
    ld_a(1, a[1]);
#pragma unroll
    for (int b = 0; b < kCB; ++b)
        bw[0][b] = dequant8(word(b, 0), sc[b], mn[b], magic);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const int cur_i = s & 1, nxt_i = cur_i ^ 1;
        if (s < 6)
            ld_a(s + 2, a[(s + 2) % 3]);
        if (s < 7) {
#pragma unroll
            for (int b = 0; b < kCB; ++b)
                bw[nxt_i][b] = dequant8(word(b, s + 1), sc[b], mn[b], magic);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int b = 0; b < kCB; ++b)
                acc[rb][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s % 3][rb], bw[cur_i][b], acc[rb][b], 0, 0, 0);
        if (s < 7) {
            // each product followed by part of the reads and vector work ahead
#pragma unroll
            for (int i = 0; i < RB * kCB; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // one product
                if (i < RB && s < 6)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // one LDS read
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);     // some vector ALU
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

// One segment of work of a workgroup: rows m0 .. m0+32*RB-1, the 256 columns
// of column group cg, chunks c_begin .. c_end-1 of K, accumulated into acc
// (zeroed here).  Wave w takes columns 32w .. 32w+31 of the group and all RB
// row blocks, so every weight is dequantised once.  Every wave of the
// workgroup calls it with the same arguments; the x ring buffers must be free
// (no wave still reading them) on entry.
template <int RB>
__device__ __forceinline__ void gemm_segment(const uint16_t *__restrict__ x, const uint8_t *__restrict__ codes,
                                             const uint16_t *__restrict__ mins,
                                             const uint16_t *__restrict__ scales, int M, int N, int K, int m0,
                                             int cg, int c_begin, int c_end, char *const (&sx)[kXBuf], int wave,
                                             int lane, f16v (&acc)[RB][kCB])
{
    const int64_t n0 = (int64_t)cg * kColsPerGroup + wave * kColsPerWave;
    const int64_t nsafe = n0 < N ? n0 : 0; // waves past N stream rows 0.. and store nothing
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int b = 0; b < kCB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                acc[rb][b][i] = 0.0f;

    // Both rings run one ring length of chunks ahead of the products: x
    // (kXBuf - 1 chunks, in LDS) and the weights (kDepth chunks, in
    // registers).  Every load is issued unconditionally, in the order
    // [x of chunk c + kXBuf - 1] [products of chunk c] [weights of chunk
    // c + kDepth] per chunk, so the x of chunk c is complete once at most
    // kWLoads (kXBuf - 1) + (x loads per chunk) (kXBuf - 2) younger loads are
    // outstanding.  The loop is unrolled by one ring length so that every
    // slot is named statically and refilled in place right after it is
    // consumed; the chunk count is padded to a multiple of it with chunks
    // that read zeros and add nothing.
    const __amdgpu_buffer_rsrc_t rx = rsrc(x, (uint32_t)((int64_t)M * K * 2));
    const WStreams wst = w_streams(codes, mins, scales, nsafe, K, lane);
    const XLoads<RB> xl = x_loads<RB>(M, K, m0, wave, lane);
    auto valid = [&](int c) { return c < c_end; };
    // prologue in the loop's own order (as if the chunks before c_begin had
    // run): W(c0) | x(c0) W(c0+1) | ..., so that every wait the compiler
    // derives for the loop body holds for the first pass as well
    WChunk w[kDepth];
    w[0] = load_w_chunk(wst, (uint32_t)c_begin, valid(c_begin));
#pragma unroll
    for (int i = 0; i < kXBuf - 1; ++i) {
        issue_x<RB>(rx, xl, (uint32_t)(c_begin + i), valid(c_begin + i), sx[i], wave);
        w[i + 1] = load_w_chunk(wst, (uint32_t)(c_begin + i + 1), valid(c_begin + i + 1));
    }
    const int n_pad = (max(c_end - c_begin, 0) + kDepth - 1) / kDepth * kDepth;
    for (int i = 0; i < n_pad; i += kDepth) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) {
            const int c = c_begin + i + u;
            // x of chunk c has landed (this wave's pieces: the wait), then every
            // wave's pieces have, and every wave is done reading the buffer the
            // next x goes into (the barrier).  One statement, no fence: a
            // workgroup fence would wait for every earlier load into LDS.
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kWLoads * (kXBuf - 1) +
                                                                  XLoads<RB>::PER_THREAD * (kXBuf - 2))
                         : "memory");
            issue_x<RB>(rx, xl, (uint32_t)(c + kXBuf - 1), valid(c + kXBuf - 1), sx[(u + kXBuf - 1) % kXBuf], wave);
            __builtin_amdgcn_sched_barrier(0);
            mma_chunk<RB>(w[u], sx[u], lane, acc);
            w[u] = load_w_chunk(wst, (uint32_t)(c + kDepth), valid(c + kDepth));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// The accumulators of a segment to memory: fp16 into y [M][N] (dst32 null),
// or binary32 into dst32, rows m0.. of a [32*RB][ld] block (ld = N for the
// split partials, 256 for a stream partial tile).  D layout: value i of lane
// l is row 8*(i/4) + 4*(l/32) + i%4 of the block, column l%32.
template <int RB>
__device__ __forceinline__ void store_segment(const f16v (&acc)[RB][kCB], _Float16 *__restrict__ y,
                                              float *__restrict__ dst32, int64_t ld32, int64_t col32, int M, int N,
                                              int m0, int cg, int wave, int lane)
{
    const int64_t n0 = (int64_t)cg * kColsPerGroup + wave * kColsPerWave;
    if (n0 >= N) // N % 64 == 0: a wave's columns are all in range or all out
        return;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int b = 0; b < kCB; ++b) {
            const int64_t n = n0 + b * 32 + (lane & 31);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = rb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                if (m0 + r < M) {
                    if (dst32 == nullptr)
                        y[(int64_t)(m0 + r) * N + n] = (_Float16)acc[rb][b][i];
                    else
                        dst32[(int64_t)r * ld32 + col32 + (n - (int64_t)cg * kColsPerGroup)] = acc[rb][b][i];
                }
            }
        }
    }
}

// Split-K form.  grid.x: column groups of 256 (fastest), grid.y: K splits,
// grid.z: row tiles of 32*RB.  splits == 1: y written as fp16; else binary32
// partials to ws[split][M][N].
template <int RB>
__global__ __launch_bounds__(kThreads, kGroupsPerCU) void k_gemm_w4(const uint16_t *__restrict__ x,
                                                         const uint8_t *__restrict__ codes,
                                                         const uint16_t *__restrict__ mins,
                                                         const uint16_t *__restrict__ scales,
                                                         _Float16 *__restrict__ y, float *__restrict__ ws, int M,
                                                         int N, int K, int chunks_per_split)
{
    // the x ring: separate arrays, so that the compiler can tell the buffer
    // being read from the ones being filled
    __shared__ __attribute__((aligned(16))) char sx0[32 * RB * kRowBytes];
    __shared__ __attribute__((aligned(16))) char sx1[32 * RB * kRowBytes];
    __shared__ __attribute__((aligned(16))) char sx2[32 * RB * kRowBytes];
    char *const sx[kXBuf] = {sx0, sx1, sx2};
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // uniform: the buffer bases stay scalar
    const int split = blockIdx.y, splits = gridDim.y;
    const int m0 = blockIdx.z * 32 * RB;
    const int c_begin = split * chunks_per_split;
    const int c_end = min(K / kChunk, c_begin + chunks_per_split);
    f16v acc[RB][kCB];
    gemm_segment<RB>(x, codes, mins, scales, M, N, K, m0, (int)blockIdx.x, c_begin, c_end, sx, wave, lane, acc);
    float *part = splits == 1 ? nullptr : ws + (int64_t)split * M * N + (int64_t)m0 * N;
    store_segment<RB>(acc, y, part, N, (int64_t)blockIdx.x * kColsPerGroup, M, N, m0, (int)blockIdx.x, wave,
                      lane);
}

// Stream form: the (tile, chunk) units -- tile t = row tile * column groups +
// column group, unit t*C + c for the C chunks of K -- are cut into gridDim.x
// equal contiguous ranges, one per workgroup (one per CU), so that no CU
// waits on a second round.  A tile covered whole by one workgroup is written
// as fp16; the part of a tile at either end of a range goes to one of that
// workgroup's two partial slots (slot 0: its first tile, slot 1: its last),
// ws [gridDim.x][2][32*RB][256] binary32, summed by k_gemm_fixup.
template <int RB>
__global__ __launch_bounds__(kThreads, kGroupsPerCU) void k_gemm_w4_stream(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ codes, const uint16_t *__restrict__ mins,
    const uint16_t *__restrict__ scales, _Float16 *__restrict__ y, float *__restrict__ ws, int M, int N, int K,
    int64_t units, int col_groups)
{
    __shared__ __attribute__((aligned(16))) char sx0[32 * RB * kRowBytes];
    __shared__ __attribute__((aligned(16))) char sx1[32 * RB * kRowBytes];
    __shared__ __attribute__((aligned(16))) char sx2[32 * RB * kRowBytes];
    char *const sx[kXBuf] = {sx0, sx1, sx2};
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int C = K / kChunk;
    const int64_t G = gridDim.x, g = blockIdx.x;
    const int64_t u0 = g * units / G, u1 = (g + 1) * units / G;
    float *const slots = ws + g * 2 * (32 * RB) * kColsPerGroup;
    int64_t u = u0;
    while (u < u1) {
        const int64_t t = u / C;
        const int c_begin = (int)(u - t * C);
        const int c_end = (int)min<int64_t>(C, u1 - t * C);
        const int cg = (int)(t % col_groups), m0 = (int)(t / col_groups) * 32 * RB;
        // the lane's offsets are recomputed for every segment rather than kept
        // live across the loop (the empty asm hides that they are invariant)
        int ln = lane;
        asm volatile("" : "+v"(ln));
        f16v acc[RB][kCB];
        gemm_segment<RB>(x, codes, mins, scales, M, N, K, m0, cg, c_begin, c_end, sx, wave, ln, acc);
        const bool whole = c_begin == 0 && c_end == C;
        float *part = whole ? nullptr : slots + (u == u0 ? 0 : 1) * (32 * RB) * kColsPerGroup;
        store_segment<RB>(acc, y, part, kColsPerGroup, 0, M, N, m0, cg, wave, ln);
        u = t * C + c_end;
        __syncthreads(); // the x ring is free (and its last loads have landed) before the next segment
    }
}

// The tiles the stream form split: y = fp16(sum of their partial slots, in
// workgroup order).  grid.x: pieces of kFixRows rows, grid.y: tiles; 256
// threads, 4 outputs each per row.  32-bit unit arithmetic: units * G < 2^32
// (checked by the host).
constexpr int kFixRows = 4;
__global__ __launch_bounds__(256) void k_gemm_fixup(const float *__restrict__ ws, _Float16 *__restrict__ y, int M,
                                                    int N, int K, uint32_t units, uint32_t G, int col_groups,
                                                    int rows)
{
    const uint32_t C = (uint32_t)(K / kChunk);
    const uint32_t t = blockIdx.y;
    auto start = [&](uint32_t g) { return g * units / G; };
    const uint32_t a = t * C, b = a + C; // the tile's units
    uint32_t g0 = a * G / units;         // the workgroup whose range holds unit a
    while (g0 + 1 < G && start(g0 + 1) <= a)
        ++g0;
    while (g0 > 0 && start(g0) > a)
        --g0;
    uint32_t g1 = g0 + 1; // one past the last workgroup with units of the tile
    while (g1 < G && start(g1) < b)
        ++g1;
    if (g1 == g0 + 1) // one workgroup covered it: written as fp16
        return;
    const int cg = (int)(t % (uint32_t)col_groups), m0 = (int)(t / (uint32_t)col_groups) * rows;
    const int col = (threadIdx.x & 63) * 4;
    const int64_t n = (int64_t)cg * kColsPerGroup + col;
    const int r = blockIdx.x * kFixRows + (threadIdx.x >> 6);
    if (r >= rows || m0 + r >= M || n >= N)
        return;
    // slot 0 of g0 holds the tile when it is g0's first tile; every later
    // workgroup starts inside the tile (slot 0)
    const float *p0 = ws + ((int64_t)(g0 * 2 + (start(g0) == a ? 0 : 1)) * rows + r) * kColsPerGroup + col;
    float4 s = *reinterpret_cast<const float4 *>(p0);
    const int64_t step = (int64_t)2 * rows * kColsPerGroup; // from slot 0 of g to slot 0 of g + 1
    const float *p = ws + ((int64_t)(g0 + 1) * 2 * rows + r) * kColsPerGroup + col;
    uint32_t g = g0 + 1;
    for (; g + 2 <= g1; g += 2, p += 2 * step) {
        const float4 v0 = *reinterpret_cast<const float4 *>(p);
        const float4 v1 = *reinterpret_cast<const float4 *>(p + step);
        s.x += v0.x;
        s.y += v0.y;
        s.z += v0.z;
        s.w += v0.w;
        s.x += v1.x;
        s.y += v1.y;
        s.z += v1.z;
        s.w += v1.w;
    }
    if (g < g1) {
        const float4 v0 = *reinterpret_cast<const float4 *>(p);
        s.x += v0.x;
        s.y += v0.y;
        s.z += v0.z;
        s.w += v0.w;
    }
    const h2 lo = {(_Float16)s.x, (_Float16)s.y}, hi = {(_Float16)s.z, (_Float16)s.w};
    *reinterpret_cast<uint2 *>(y + (int64_t)(m0 + r) * N + n) =
        make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
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

template <int RB>
int launch_gemm_rb(const GemmArgs &g, hipStream_t st)
{
    const int col_groups = (g.N + kColsPerGroup - 1) / kColsPerGroup;
    const int row_tiles = (g.M + 32 * RB - 1) / (32 * RB);
    if (g.splits == 0) { // stream form
        const int64_t units = (int64_t)col_groups * row_tiles * (g.K / kChunk);
        hipLaunchKernelGGL((k_gemm_w4_stream<RB>), dim3((unsigned)g.stream_groups), dim3(kThreads), 0, st,
                           static_cast<const uint16_t *>(g.x), g.codes, static_cast<const uint16_t *>(g.mins),
                           static_cast<const uint16_t *>(g.scales), static_cast<_Float16 *>(g.y), g.ws, g.M, g.N,
                           g.K, units, col_groups);
        int e = (int)hipGetLastError();
        if (e != 0)
            return e;
        hipLaunchKernelGGL(k_gemm_fixup, dim3((unsigned)(32 * RB / kFixRows), (unsigned)(col_groups * row_tiles)),
                           dim3(256), 0, st, g.ws,
                           static_cast<_Float16 *>(g.y), g.M, g.N, g.K, (uint32_t)units, (uint32_t)g.stream_groups,
                           col_groups, 32 * RB);
        return (int)hipGetLastError();
    }
    const dim3 grid((unsigned)col_groups, (unsigned)g.splits, (unsigned)row_tiles);
    hipLaunchKernelGGL((k_gemm_w4<RB>), grid, dim3(kThreads), 0, st, static_cast<const uint16_t *>(g.x), g.codes,
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

// Row blocks of 32 per row tile: up to 5 (160 rows; M = 144 pads 16 rows).
int gemm_row_blocks(int M) { return M > 128 ? 5 : (M + 31) / 32; }

int launch_gemm_w4(const GemmArgs &g, hipStream_t st)
{
    switch (gemm_row_blocks(g.M)) {
    case 1: return launch_gemm_rb<1>(g, st);
    case 2: return launch_gemm_rb<2>(g, st);
    case 3: return launch_gemm_rb<3>(g, st);
    case 4: return launch_gemm_rb<4>(g, st);
    default: return launch_gemm_rb<5>(g, st);
    }
}

} // namespace kvq
