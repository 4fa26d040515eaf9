// fp8.hip -- the FP8 second stage: h quantised to MX FP8 (E4M3 codes, one E8M0 scale per 32 values
// along I) and the down product y = h . Wd_e^T on gfx950's scaled MX matrix-core instruction
// (16x16x128, FP8 x FP4 with one E8M0 scale per operand row and 32-input block, FP32 accumulate),
// which consumes the E4M3 codes and the MXFP4 weight codes with their scales as they are: no
// conversion to BF16 on either side.
//
// Operand layout of the scaled 16x16x128 instruction (one wave; lane l, g = l / 16):
//  * an FP4 operand is 4 dwords: row (or column) l % 16, inputs 32 g .. 32 g + 31, element 2i in
//    the low nibble of byte i;
//  * an FP8 operand is 8 dwords: row l % 16, bytes 0..15 = inputs 16 g .. 16 g + 15 and bytes
//    16..31 = inputs 64 + 16 g .. 64 + 16 g + 15;
//  * each operand's scale argument is lane l's E8M0 byte for row l % 16 and input block g
//    (inputs 32 g .. 32 g + 31), whichever lane holds those inputs.
// MX8 weight blocks (16 rows x 128 inputs, 1088 bytes, same count and order as the MX blocks of
// common.hpp): bytes [16 l, 16 l + 16) are lane l's FP4 operand, byte 1024 + l its scale.
#include "kernels.hpp"

#include <algorithm>

namespace mxmoe {

typedef int v8i32_t __attribute__((ext_vector_type(8)));

// Scaled MX product, operand formats fixed at compile time (0 = FP8 E4M3, 4 = FP4 E2M1).
template <int FA, int FB>
__device__ inline f32x4_t mfma_mx(v8i32_t a, v8i32_t b, uint32_t sa, uint32_t sb, f32x4_t c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, (int)sa, 0, (int)sb);
}

__device__ inline v8i32_t fp8_operand(u32x4_t lo, u32x4_t hi)
{
    return v8i32_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
__device__ inline v8i32_t fp4_operand(u32x4_t c)
{
    return v8i32_t{(int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0, 0, 0};
}

// ---------------------------------------------------------------------------------------------
// Packing: canonical down codes [E, N, K/2] / scales [E, N, K/32] -> MX8 blocks. One thread per
// (block, lane): 16 code bytes (row nb*16 + l%16, inputs kb*128 + 32 (l/16) ..) and one scale byte.
__global__ void pack_mx8_kernel(uint8_t *__restrict__ dst, const uint8_t *__restrict__ codes,
                                const uint8_t *__restrict__ scales, int64_t E, int64_t N, int64_t K)
{
    const int64_t chunk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t kblocks = K / MX_STEP, nblocks = N / 16;
    if (chunk >= E * nblocks * kblocks * WAVE)
        return;
    const int lane = (int)(chunk % WAVE);
    const int64_t blk = chunk / WAVE;                 // = (e * nblocks + nb) * kblocks + kb
    const int64_t e = blk / (nblocks * kblocks);
    const int64_t nb = (blk / kblocks) % nblocks, kb = blk % kblocks;
    const int64_t row = nb * 16 + (lane & 15), g = lane >> 4;
    const uint8_t *src = codes + (e * N + row) * (K / 2) + (kb * MX_STEP + 32 * g) / 2;
    u32x4_t v;
    for (int j = 0; j < 4; j++)
        v[j] = *reinterpret_cast<const uint32_t *>(src + 4 * j);
    uint8_t *out = dst + blk * MX_BLOCK_BYTES;
    *reinterpret_cast<u32x4_t *>(out + lane * 16) = v;
    out[MX_CODE_BYTES + lane] = scales[(e * N + row) * (K / 32) + kb * 4 + g];
}

hipError_t launch_pack_down8(uint8_t *dst, const uint8_t *dc, const uint8_t *ds, int64_t E, int64_t I, int64_t Lt,
                             hipStream_t st)
{
    if (Lt % 16 || I % MX_STEP)
        return hipErrorInvalidValue;
    const int64_t threads = E * (Lt / 16) * (I / MX_STEP) * WAVE;
    if (threads <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(pack_mx8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, dst, dc, ds, E,
                       Lt, I);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// MX FP8 quantisation of h (rows of I BF16 values). Each lane converts 8 consecutive values; the
// four lanes of one 32-value block exchange their largest magnitude, so the block scale is
// X = floor(log2 max|h|) - 8, clamped to [-127, 127] (-127 for an all-zero block). Each element
// h / 2^X is rounded to nearest even at E4M3 precision in integer arithmetic, exactly: a BF16
// value is S 2^E0 with an integer significand S < 256, so the quotient's bits are S's bits.

// E4M3 code of the BF16 value `b` divided by 2^X: round to nearest even, saturate at 448,
// keep the sign bit.
__device__ inline uint32_t e4m3_code(uint32_t b, int X)
{
    const uint32_t sign = (b >> 8) & 0x80u, mag = b & 0x7FFFu;
    if (mag == 0u)
        return sign;
    const uint32_t eb = mag >> 7, m = mag & 0x7Fu;
    const uint32_t S = eb ? (0x80u | m) : m;          // value = S 2^E0
    const int E0 = eb ? (int)eb - 134 : -133;
    const int L = 31 - __builtin_clz(S);              // leading bit of S
    const int Eq = L + E0 - X;                        // exponent of the quotient's leading bit
    const int qe = max(Eq - 3, -9);                   // quantum: 4 significant bits, or 2^-9
    const int sh = qe - (E0 - X);                     // low bits of S below the quantum
    uint32_t r;
    if (sh <= 0) {
        r = S << (-sh);
    } else if (sh > 9) {
        r = 0u;                                       // below half the quantum (S < 2^8)
    } else {
        r = S >> sh;
        const uint32_t rem = S & ((1u << sh) - 1u), half = 1u << (sh - 1);
        r += (rem > half || (rem == half && (r & 1u))) ? 1u : 0u;
    }
    // value r 2^qe with r in [8, 16] (or < 8 at qe = -9): code (qe + 9) 8 + r, capped at 448
    const int code = min((qe + 9) * 8 + (int)r, 0x7E);
    return sign | (uint32_t)code;
}

__global__ void fp8_quant_kernel(const uint16_t *__restrict__ h, int64_t n8, uint8_t *__restrict__ codes,
                                 uint8_t *__restrict__ scales)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // 8-value group
    const bool live = i < n8;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (live)
        v = load16(h + i * 8);
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        amax = max(amax, v[j] & 0x7FFFu);
        amax = max(amax, (v[j] >> 16) & 0x7FFFu);
    }
    // the four lanes of a 32-value block are lanes 4k .. 4k+3 (n8 is a multiple of 4)
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
    if (!live)
        return;
    const int X = amax ? min(max(bf16_ilogb(amax) - 8, -127), 127) : -127;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 2; j++) {
        lo |= e4m3_code(v[j] & 0xFFFFu, X) << (16 * j);
        lo |= e4m3_code(v[j] >> 16, X) << (16 * j + 8);
        hi |= e4m3_code(v[j + 2] & 0xFFFFu, X) << (16 * j);
        hi |= e4m3_code(v[j + 2] >> 16, X) << (16 * j + 8);
    }
    *reinterpret_cast<uint2 *>(codes + i * 8) = make_uint2(lo, hi);
    if ((i & 3) == 0)
        scales[i >> 2] = (uint8_t)(X + 127);
}

hipError_t launch_fp8_quant(const uint16_t *h, int64_t rows, int64_t I, uint8_t *codes, uint8_t *scales,
                            hipStream_t st)
{
    if (I % 32 || rows < 0)
        return hipErrorInvalidValue;
    const int64_t n8 = rows * I / 8;
    if (n8 == 0)
        return hipSuccess;
    if ((n8 + 255) / 256 > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(fp8_quant_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, h, n8, codes, scales);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Down product for expert tiles of at most 16 rows (few tokens per expert): the time is the HBM
// stream of the MX8 weights. One wave per 64 output columns (four 16-row weight blocks) and tile;
// it issues the weight, activation and scale loads of every 128-input block of its K range (up to
// MAXS blocks at a time, addresses clamped into range so no load is conditional), then multiplies.
// A = the FP8 rows of h (scaled-instruction operand A), B = the weights (operand B): lane l's
// accumulators are rows 4 (l/16) + i, column l % 16 of a 16 x 16 fragment.
template <int NT, int MAXS>
__global__ __launch_bounds__(WAVE) void down8_stream_kernel(const Fp8DownArgs g)
{
    constexpr int BN = 16 * NT;
    const int lane = threadIdx.x;
    if ((int)blockIdx.y >= g.tiles[0])
        return;
    const int4 tile = reinterpret_cast<const int4 *>(g.tiles + TILE_HEADER_INTS)[blockIdx.y];
    const int group = tile.x, m0 = tile.y, m1 = tile.z;
    const int n0 = blockIdx.x * BN;

    const int r = m0 + (lane & 15), q = lane >> 4;
    const bool aval = r < m1;
    const uint8_t *arow = g.codes + (int64_t)(aval ? r : m0) * g.K + 16 * q;
    const uint8_t *srow = g.scales + (int64_t)(aval ? r : m0) * (g.K / 32) + q;
    const int nblk = g.K / MX_STEP;
    const uint8_t *Bg = g.B + (int64_t)group * g.b_stride;

    f32x4_t acc[NT];
#pragma unroll
    for (int nf = 0; nf < NT; nf++)
        acc[nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const u32x4_t zero4 = {0u, 0u, 0u, 0u};

    for (int kb = 0; kb < nblk; kb += MAXS) {
        const int cnt = min(MAXS, nblk - kb);
        u32x4_t codes[MAXS][NT];
        uint32_t sc[MAXS][NT];
        u32x4_t alo[MAXS], ahi[MAXS];
        uint32_t as[MAXS];
#pragma unroll
        for (int s = 0; s < MAXS; s++) {
            const int blk = kb + min(s, cnt - 1);
#pragma unroll
            for (int nf = 0; nf < NT; nf++) {
                const uint8_t *p = Bg + ((int64_t)(n0 / 16 + nf) * nblk + blk) * MX_BLOCK_BYTES;
                codes[s][nf] = load16_nt(p + lane * 16);
                sc[s][nf] = p[MX_CODE_BYTES + lane];
            }
        }
#pragma unroll
        for (int s = 0; s < MAXS; s++) {
            const int blk = kb + min(s, cnt - 1);
            alo[s] = aval ? load16(arow + blk * MX_STEP) : zero4;
            ahi[s] = aval ? load16(arow + blk * MX_STEP + 64) : zero4;
            as[s] = srow[blk * 4];
        }
#pragma unroll
        for (int s = 0; s < MAXS; s++) {
            if (s < cnt) {
                const v8i32_t a = fp8_operand(alo[s], ahi[s]);
#pragma unroll
                for (int nf = 0; nf < NT; nf++)
                    acc[nf] = mfma_mx<0, 4>(a, fp4_operand(codes[s][nf]), as[s], sc[s][nf], acc[nf]);
            }
        }
    }

    uint16_t *out = g.out;
#pragma unroll
    for (int nf = 0; nf < NT; nf++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int rr = m0 + 4 * q + i, n = n0 + nf * 16 + (lane & 15);
            if (rr < m1)
                out[(int64_t)rr * g.ldo + n] = (uint16_t)f32_to_bf16_bits(acc[nf][i]);
        }
}

// ---------------------------------------------------------------------------------------------
// A-stationary down product for many rows per expert. The workgroup stages its 128-row FP8 tile
// of h (128 x K bytes, at most 64 KiB) into LDS once with direct global->LDS loads, as whole
// 128-byte lines (see astat8_item). It then walks its
// run of 256-column N blocks; each of the four waves owns 128 x 64 outputs per N block. The
// weights are operand A of the scaled instruction (FP4, rows = output columns) and h operand B
// (FP8, columns = rows of h), so lane (q, c) of a fragment holds four consecutive output columns
// 4q .. 4q+3 of row c. The outputs leave through a 2 KiB LDS staging area per wave, one 16-row
// fragment at a time, so that every store instruction writes whole 128-byte row segments (stores
// of 32-byte pieces at the 7 KiB row stride ran at a quarter of the rate). Weights are loaded one
// 128-input block ahead (across N blocks too).
constexpr int A8_WAVES = 4, A8_BN = A8_WAVES * 64, A8_MF = 8, A8_NF = 4, A8_XCDS = 8;
constexpr int A8_STAGE_PITCH = 144;                      // bytes per staged row (128 + 16 padding)
constexpr int A8_STAGE_BYTES = 16 * A8_STAGE_PITCH;       // one 16-row fragment of one wave

template <int KB, int NMF>
__device__ __attribute__((always_inline)) inline void astat8_item(const Fp8DownArgs &g, int group, int m0, int m1,
                                                                  int j0, int j1, u32x4_t *lds, uint8_t *stage_all)
{
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const int q = lane >> 4;
    uint8_t *stage = stage_all + wv * A8_STAGE_BYTES;

    // As whole 128-byte lines: row-half h of fragment f, block kb is one 1 KiB block at
    // (f * KB + kb) * 2 + h, 8 rows x 128 bytes, row r8's 16-byte chunk c at position c ^ r8 (the
    // operand reads, rows 0..7 of one chunk at a time, fall in distinct banks). Operand-order blocks
    // of 16 rows x 64 bytes, half a line each, stream from L2 at about a third of the rate.
    for (int b = wv; b < KB * 2 * NMF; b += A8_WAVES) {
        const int f = b % NMF, kb = (b / NMF) / 2, h = (b / NMF) % 2, r8 = lane >> 3;
        const int r = min(m0 + f * 16 + h * 8 + r8, m1 - 1);   // clamped valid row, never stored
        __builtin_amdgcn_global_load_lds(g.codes + (int64_t)r * g.K + kb * MX_STEP + 16 * ((lane & 7) ^ r8),
                                         (__attribute__((address_space(3))) void *)&lds[((f * KB + kb) * 2 + h) * WAVE],
                                         16, 0, 0);
    }
    // h scales: lane l needs row f*16 + l%16, block kb*4 + l/16, one byte per kb
    uint32_t hsc[NMF];
#pragma unroll
    for (int f = 0; f < NMF; f++) {
        const int r = min(m0 + f * 16 + (lane & 15), m1 - 1);
        const uint8_t *sp = g.scales + (int64_t)r * (g.K / 32) + q;
        uint32_t v = 0;
#pragma unroll
        for (int kb = 0; kb < KB; kb++)
            v |= (uint32_t)sp[kb * 4] << (8 * kb);
        hsc[f] = v;
    }

    const uint8_t *Bg = g.B + (int64_t)group * g.b_stride;
    const int nbmax = g.N / 16 - 1;
    // cached loads: every tile of an expert reads the expert's whole matrix
    auto load_kb = [&](int j, int kb, u32x4_t *codes, uint32_t *sc) {
#pragma unroll
        for (int nf = 0; nf < A8_NF; nf++) {
            const int nb = min((j * A8_BN + wv * 64) / 16 + nf, nbmax);
            const uint8_t *p = Bg + ((int64_t)nb * KB + kb) * MX_BLOCK_BYTES;
            codes[nf] = load16(p + lane * 16);
            sc[nf] = p[MX_CODE_BYTES + lane];
        }
    };
    u32x4_t bc[A8_NF];
    uint32_t bs[A8_NF];
    load_kb(j0, 0, bc, bs);
    __builtin_amdgcn_s_waitcnt(0);                                // A tile, scales and first B landed
    __syncthreads();

    uint16_t *out = g.out;
    for (int j = j0; j < j1; j++) {
        f32x4_t acc[NMF][A8_NF];
#pragma unroll
        for (int f = 0; f < NMF; f++)
#pragma unroll
            for (int nf = 0; nf < A8_NF; nf++)
                acc[f][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int kb = 0; kb < KB; kb++) {
            u32x4_t bn[A8_NF];
            uint32_t bsn[A8_NF];
            if (kb + 1 < KB)
                load_kb(j, kb + 1, bn, bsn);
            else
                load_kb(min(j + 1, j1 - 1), 0, bn, bsn);
            // h operands one fragment ahead of their use, so that only two are live at a time: lane
            // (q, c) takes chunks q and 4 + q (inputs 16 q .., 64 + 16 q ..) of row c of the fragment
            const int ar = lane & 15;
            const int alo_at = (ar >> 3) * WAVE + (ar & 7) * 8 + (q ^ (ar & 7));
            const int ahi_at = (ar >> 3) * WAVE + (ar & 7) * 8 + ((4 + q) ^ (ar & 7));
            u32x4_t alo = lds[(kb * 2) * WAVE + alo_at], ahi = lds[(kb * 2) * WAVE + ahi_at];
#pragma unroll
            for (int f = 0; f < NMF; f++) {
                const v8i32_t a = fp8_operand(alo, ahi);
                if (f + 1 < NMF) {
                    alo = lds[((f + 1) * KB + kb) * 2 * WAVE + alo_at];
                    ahi = lds[((f + 1) * KB + kb) * 2 * WAVE + ahi_at];
                }
                const uint32_t sa = (hsc[f] >> (8 * kb)) & 0xFFu;
#pragma unroll
                for (int nf = 0; nf < A8_NF; nf++)
                    acc[f][nf] = mfma_mx<4, 0>(fp4_operand(bc[nf]), a, bs[nf], sa, acc[f][nf]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int nf = 0; nf < A8_NF; nf++) {
                bc[nf] = bn[nf];
                bs[nf] = bsn[nf];
            }
        }
        // Output through this wave's LDS staging area, one 16-row fragment at a time: lane (q, c)
        // puts row c, columns nf*16 + 4q .. +3 in; then each lane takes 8 consecutive columns of
        // one row, so a store instruction writes eight whole 128-byte row segments.
        // Rows past the tile end, and a column slice past N, fall outside the store window.
        const int n0w = j * A8_BN + wv * 64;
        const int wrows = n0w < g.N ? min(m1 - m0, NMF * 16) : 0;
        const auto win = row_window(wrows > 0 ? out + (int64_t)m0 * g.ldo + n0w : out, wrows, g.ldo);
#pragma unroll
        for (int f = 0; f < NMF; f++) {
#pragma unroll
            for (int nf = 0; nf < A8_NF; nf++)
                *reinterpret_cast<uint2 *>(stage + (lane & 15) * A8_STAGE_PITCH + nf * 32 + 8 * q) =
                    make_uint2(pack_bf16x2(acc[f][nf][0], acc[f][nf][1]),
                               pack_bf16x2(acc[f][nf][2], acc[f][nf][3]));
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int rr = h * 8 + (lane >> 3);
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(stage + rr * A8_STAGE_PITCH + (lane & 7) * 16);
                store16_window<CPOL_NT>(v, win, ((f * 16 + rr) * g.ldo + (lane & 7) * 8) * 2);
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

template <int KB>
__global__ __launch_bounds__(WAVE * A8_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void astat8_kernel(const Fp8DownArgs g, int nsplit)
{
    __shared__ u32x4_t lds[KB * 2 * A8_MF * WAVE];
    __shared__ __attribute__((aligned(16))) uint8_t stage[A8_WAVES * A8_STAGE_BYTES];
    const int total = g.tiles[0] * nsplit;
    const int per = (total + A8_XCDS - 1) / A8_XCDS;
    const int slot = blockIdx.x / A8_XCDS;
    const int item = (blockIdx.x % A8_XCDS) * per + slot;
    if (slot >= per || item >= total)
        return;
    const int4 t = reinterpret_cast<const int4 *>(g.tiles + TILE_HEADER_INTS)[item / nsplit];
    const int part = item % nsplit;
    const int nbn = (g.N + A8_BN - 1) / A8_BN;
    const int j0 = part * nbn / nsplit, j1 = (part + 1) * nbn / nsplit;
    if (j0 >= j1)
        return;
    const int nmf = __builtin_amdgcn_readfirstlane((t.z - t.y + 15) / 16);
    if (nmf <= 2)
        astat8_item<KB, 2>(g, t.x, t.y, t.z, j0, j1, lds, stage);
    else if (nmf <= 4)
        astat8_item<KB, 4>(g, t.x, t.y, t.z, j0, j1, lds, stage);
    else
        astat8_item<KB, 8>(g, t.x, t.y, t.z, j0, j1, lds, stage);
}

template <int KB>
static hipError_t launch_astat8_t(const Fp8DownArgs &g, int max_tiles, hipStream_t st)
{
    const int nbn = (g.N + A8_BN - 1) / A8_BN;
    const int nsplit = std::max(1, std::min(nbn, (2048 + max_tiles - 1) / max_tiles));
    const int64_t items = (int64_t)max_tiles * nsplit;
    const int64_t grid = (items + A8_XCDS - 1) / A8_XCDS * A8_XCDS;
    if (grid > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((astat8_kernel<KB>), dim3((unsigned)grid), dim3(WAVE * A8_WAVES), 0, st, g, nsplit);
    return hipGetLastError();
}

hipError_t launch_down_fp8(const Fp8DownArgs &g, bool many_rows, int max_tiles, hipStream_t st)
{
    if (!g.tiles || !g.codes || !g.scales || !g.B || !g.out || g.N <= 0 || g.N % 64 || g.K < MX_STEP ||
        g.K % MX_STEP || g.K > FP8_DOWN_MAX_K || g.ldo < g.N || g.ldo % 8 ||
        reinterpret_cast<uintptr_t>(g.codes) % 16 || reinterpret_cast<uintptr_t>(g.out) % 16)
        return hipErrorInvalidValue;
    if (max_tiles <= 0)
        return hipSuccess;
    if (!many_rows) {
        if (max_tiles > 65535)
            return hipErrorInvalidValue;
        // blocks per batch: all of them up to four, else 4 or 3 when that divides the count, so that
        // no batch re-reads a clamped block (a repeated fourth block at K = 384 cost 12%)
        const int nblk = g.K / MX_STEP;
        const int batch = nblk <= 4 ? nblk : nblk % 3 == 0 && nblk % 4 != 0 ? 3 : 4;
        const dim3 grid(g.N / 64, max_tiles);
        if (batch == 4)
            hipLaunchKernelGGL((down8_stream_kernel<4, 4>), grid, dim3(WAVE), 0, st, g);
        else if (batch == 3)
            hipLaunchKernelGGL((down8_stream_kernel<4, 3>), grid, dim3(WAVE), 0, st, g);
        else if (batch == 2)
            hipLaunchKernelGGL((down8_stream_kernel<4, 2>), grid, dim3(WAVE), 0, st, g);
        else
            hipLaunchKernelGGL((down8_stream_kernel<4, 1>), grid, dim3(WAVE), 0, st, g);
        return hipGetLastError();
    }
    switch (g.K / MX_STEP) {
    case 1: return launch_astat8_t<1>(g, max_tiles, st);
    case 2: return launch_astat8_t<2>(g, max_tiles, st);
    case 3: return launch_astat8_t<3>(g, max_tiles, st);
    case 4: return launch_astat8_t<4>(g, max_tiles, st);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mxmoe
