// fp4.hip -- the A4W4 first stage: the latent activations z quantised to MX FP4 (E2M1 codes, one
// E8M0 scale per 32 values along Lt) and the grouped gate|up product with the GLU on gfx950's scaled
// MX matrix-core instruction (16x16x128, FP4 x FP4, one E8M0 scale per operand row and 32-input
// block, FP32 accumulate), which takes the activation codes and the weight codes with both scale
// vectors as they are.
//
// Operand layout of the scaled 16x16x128 instruction with FP4 operands (one wave; lane l,
// g = l / 16): 4 dwords holding row (or column) l % 16, inputs 32 g .. 32 g + 31, element 2i in the
// low nibble of byte i; the scale argument is lane l's E8M0 byte for that row and input block.
// A4 weight blocks (16 rows x 128 inputs, 1088 bytes, the count and order of the MX blocks of
// common.hpp, gate and up rows interleaved per 16): bytes [16 l, 16 l + 16) are lane l's operand,
// byte 1024 + l its scale.
#include "kernels.hpp"

#include <algorithm>

namespace mxmoe {

typedef int v8i32_t __attribute__((ext_vector_type(8)));

__device__ inline v8i32_t fp4_operand8(u32x4_t c)
{
    return v8i32_t{(int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0, 0, 0};
}

// ---------------------------------------------------------------------------------------------
// Packing: canonical gate / up codes [E, I, Lt/2] and scales [E, I, Lt/32] -> A4 blocks. Row block
// nb of the 2I interleaved rows is gate rows 16 (nb / 2) .. when nb is even, up rows when odd. One
// thread per (block, lane): 16 code bytes (row l % 16, inputs kb*128 + 32 (l / 16) ..) and one scale.
__global__ void pack_gateup4_kernel(uint8_t *__restrict__ dst, const uint8_t *__restrict__ gc,
                                    const uint8_t *__restrict__ gs, const uint8_t *__restrict__ uc,
                                    const uint8_t *__restrict__ us, int64_t E, int64_t I, int64_t Lt)
{
    const int64_t chunk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t kblocks = Lt / MX_STEP, nblocks = 2 * I / 16;
    if (chunk >= E * nblocks * kblocks * WAVE)
        return;
    const int lane = (int)(chunk % WAVE);
    const int64_t blk = chunk / WAVE;                 // = (e * nblocks + nb) * kblocks + kb
    const int64_t e = blk / (nblocks * kblocks);
    const int64_t nb = (blk / kblocks) % nblocks, kb = blk % kblocks;
    const uint8_t *codes = (nb & 1) ? uc : gc;
    const uint8_t *scales = (nb & 1) ? us : gs;
    const int64_t row = (nb >> 1) * 16 + (lane & 15), g = lane >> 4;
    const uint8_t *src = codes + (e * I + row) * (Lt / 2) + kb * (MX_STEP / 2) + 16 * g;
    u32x4_t v;
    for (int j = 0; j < 4; j++)
        v[j] = *reinterpret_cast<const uint32_t *>(src + 4 * j);
    uint8_t *out = dst + blk * MX_BLOCK_BYTES;
    *reinterpret_cast<u32x4_t *>(out + lane * 16) = v;
    out[MX_CODE_BYTES + lane] = scales[(e * I + row) * (Lt / 32) + kb * 4 + g];
}

hipError_t launch_pack_gateup4(uint8_t *dst, const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                               const uint8_t *us, int64_t E, int64_t I, int64_t Lt, hipStream_t st)
{
    if (I % 16 || Lt % MX_STEP)
        return hipErrorInvalidValue;
    const int64_t threads = E * (2 * I / 16) * (Lt / MX_STEP) * WAVE;
    if (threads <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(pack_gateup4_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, dst, gc, gs, uc,
                       us, E, I, Lt);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// MX FP4 quantisation of z (rows of L BF16 values). Each lane converts 8 consecutive values into 4
// code bytes; the four lanes of one 32-value block exchange their largest magnitude, so the block
// scale is X = floor(log2 max|z|) - 2, clamped to [-127, 127] (-127 for an all-zero block). Each
// element z / 2^X is rounded to nearest even at E2M1 precision in integer arithmetic, exactly: a
// BF16 value is S 2^E0 with an integer significand S < 256, so the quotient's bits are S's bits.

// E2M1 code of the BF16 value `b` divided by 2^X: round to nearest even, saturate at 6, keep the
// sign bit (bit 3).
__device__ inline uint32_t e2m1_code(uint32_t b, int X)
{
    const uint32_t sign = (b >> 12) & 0x8u, mag = b & 0x7FFFu;
    if (mag == 0u)
        return sign;
    const uint32_t eb = mag >> 7, m = mag & 0x7Fu;
    const uint32_t S = eb ? (0x80u | m) : m;          // value = S 2^E0
    const int E0 = eb ? (int)eb - 134 : -133;
    const int L = 31 - __builtin_clz(S);              // leading bit of S
    const int Eq = L + E0 - X;                        // exponent of the quotient's leading bit
    const int qe = max(Eq - 1, -1);                   // quantum: 2 significant bits, or 1/2
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
    // value r 2^qe: code r at qe = -1 (r in 0..4), 2 qe + 2 + r above (r in 2..4), capped at 6.0
    const int code = min(2 * qe + 2 + (int)r, 7);
    return sign | (uint32_t)code;
}

__global__ void fp4_quant_kernel(const uint16_t *__restrict__ z, int64_t n8, uint8_t *__restrict__ codes,
                                 uint8_t *__restrict__ scales)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // 8-value group
    const bool live = i < n8;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (live)
        v = load16(z + i * 8);
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
    const int X = amax ? min(max(bf16_ilogb(amax) - 2, -127), 127) : -127;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; j++)
        w |= (e2m1_code(v[j] & 0xFFFFu, X) | (e2m1_code(v[j] >> 16, X) << 4)) << (8 * j);
    *reinterpret_cast<uint32_t *>(codes + i * 4) = w;
    if ((i & 3) == 0)
        scales[i >> 2] = (uint8_t)(X + 127);
}

hipError_t launch_fp4_quant(const uint16_t *z, int64_t rows, int64_t L, uint8_t *codes, uint8_t *scales,
                            hipStream_t st)
{
    if (L % 32 || rows < 0)
        return hipErrorInvalidValue;
    const int64_t n8 = rows * L / 8;
    if (n8 == 0)
        return hipSuccess;
    if ((n8 + 255) / 256 > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(fp4_quant_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, z, n8, codes, scales);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Grouped gate|up product with the GLU on MX FP4 z. Each workgroup computes one expert tile (up to
// 128 rows, gathered through the expert-sorted pair order) times 256 of the 2I interleaved gate /
// up columns; each of its four waves owns 64 columns (four 16-row weight blocks: gate, up, gate,
// up) for every row fragment of the tile. K advances in 256-input stages (two MX blocks):
//  * A (the tile's FP4 rows and their scale dwords) is moved into LDS by direct global->LDS loads,
//    one stage ahead, into two alternating buffers. A stage of one row is one whole 128-byte line
//    of codes; a load instruction moves eight such lines (lane l: row l / 8, 16-byte chunk
//    (l % 8) ^ (row % 8), so that the reads below are conflict-free), which keeps every request a
//    whole line (half lines are served at a third of the rate from L2). Scales: per 16-row
//    fragment one load of the two scale dwords of every row (lane l: row l % 16, dword (l / 16) % 2);
//  * B (the weights' A4 blocks, two per stage) is loaded into registers one stage ahead.
// The weights are operand A of the scaled instruction (rows = output columns) and z operand B, so
// lane (q, c) of a fragment holds token row c and the four columns 4q .. 4q + 3: the GLU pairs a
// gate fragment with the up fragment beside it. Work is mapped XCD-major (the column blocks of a
// tile, then the next tile of the same expert, on one XCD). A K that is an odd number of MX blocks
// ends with a half stage: its second half re-reads valid bytes and its products are skipped.
constexpr int A4_WAVES = 4, A4_BN = A4_WAVES * 64, A4_MF = 8, A4_NF = 4, A4_XCDS = 8;

struct A4Lds {
    u32x4_t codes[2][A4_MF][2][WAVE];   // [buffer][fragment][row half: 8 lines of 8 chunks]
    uint32_t scales[2][A4_MF][WAVE];
};

template <int NMF>
__device__ __attribute__((always_inline)) inline void a4_tile(const A4GateupArgs &g, int bx, int group, int m0,
                                                              int m1, A4Lds &lds)
{
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const int n0 = bx * A4_BN + wv * 64;                          // this wave's first column
    const int nblocks = g.N / 16;
    const int kblocks = g.K / MX_STEP;
    const int nst = (kblocks + 1) / 2;
    const int row_bytes = g.K / 2;
    const uint8_t *Bg = g.B + (int64_t)group * g.b_stride;

    // Loads of a stage: 2 NMF half fragments of codes (eight lines each) and NMF scale blocks.
    // Wave wv takes items wv + 4u; with fewer items than waves the spare waves repeat one, and past
    // the last item a load repeats the last one (the same bytes into the same LDS slots), so every
    // wave issues the same number of loads on every path and the waits stay exact.
    constexpr int CC = (2 * NMF + A4_WAVES - 1) / A4_WAVES, CS = (NMF + A4_WAVES - 1) / A4_WAVES;
    const uint8_t *csrc[CC], *ssrc[CS];
    int cslot[CC], sslot[CS];
    bool chi[CC];
    const int r8 = lane >> 3, cpos = (lane & 7) ^ r8;            // logical chunk this lane moves
#pragma unroll
    for (int u = 0; u < CC; u++) {
        const int b = 2 * NMF >= A4_WAVES ? min(wv + A4_WAVES * u, 2 * NMF - 1) : wv % (2 * NMF);
        const int r = min(m0 + (b >> 1) * 16 + (b & 1) * 8 + r8, m1 - 1);   // clamped valid row, never stored
        const int64_t row = g.a_index ? (int64_t)(g.a_index[r] / g.a_div) : (int64_t)r;
        csrc[u] = g.zq + row * row_bytes + 16 * cpos;
        cslot[u] = b;
        chi[u] = cpos >= 4;
    }
#pragma unroll
    for (int u = 0; u < CS; u++) {
        const int f = NMF >= A4_WAVES ? min(wv + A4_WAVES * u, NMF - 1) : wv % NMF;
        const int r = min(m0 + f * 16 + (lane & 15), m1 - 1);
        const int64_t row = g.a_index ? (int64_t)(g.a_index[r] / g.a_div) : (int64_t)r;
        ssrc[u] = g.zs + row * (g.K / 32) + 4 * ((lane >> 4) & 1);
        sslot[u] = f;
    }
    auto issue_a = [&](int stage, int buf) {
        // the second half of a final half stage re-reads the first half (in bounds, never used)
        const bool half = 2 * stage + 1 >= kblocks;
#pragma unroll
        for (int u = 0; u < CC; u++)
            __builtin_amdgcn_global_load_lds(csrc[u] + stage * 128 - (half && chi[u] ? 64 : 0),
                                             (__attribute__((address_space(3))) void *)&lds.codes[buf][cslot[u] >> 1]
                                                                                                   [cslot[u] & 1][0],
                                             16, 0, 0);
#pragma unroll
        for (int u = 0; u < CS; u++)
            __builtin_amdgcn_global_load_lds(ssrc[u] + stage * 8 - (half && (lane & 16) ? 4 : 0),
                                             (__attribute__((address_space(3))) void *)&lds.scales[buf][sslot[u]][0], 4,
                                             0, 0);
    };
    auto load_b = [&](int stage, u32x4_t (*codes)[A4_NF], uint32_t (*sc)[A4_NF]) {
#pragma unroll
        for (int s = 0; s < 2; s++) {
            const int kb = min(2 * stage + s, kblocks - 1);
#pragma unroll
            for (int nf = 0; nf < A4_NF; nf++) {
                const int nb = min(n0 / 16 + nf, nblocks - 1);
                const uint8_t *p = Bg + ((int64_t)nb * kblocks + kb) * MX_BLOCK_BYTES;
                codes[s][nf] = load16(p + lane * 16);
                sc[s][nf] = p[MX_CODE_BYTES + lane];
            }
        }
    };

    f32x4_t acc[NMF][A4_NF];
#pragma unroll
    for (int f = 0; f < NMF; f++)
#pragma unroll
        for (int nf = 0; nf < A4_NF; nf++)
            acc[f][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // the first B before the first A stage, so that the prologue's full wait covers both
    u32x4_t bcur[2][A4_NF];
    uint32_t scur[2][A4_NF];
    load_b(0, bcur, scur);
    issue_a(0, 0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int q = lane >> 4, ar = lane & 15, rh = ar >> 3, rl = ar & 7;
    for (int st = 0; st < nst; st++) {
        const int cur = st & 1;
        issue_a(min(st + 1, nst - 1), cur ^ 1);   // before this stage's B prefetch (vmcnt order)
        asm volatile("" ::: "memory");
        u32x4_t bnx[2][A4_NF];
        uint32_t snx[2][A4_NF];
        load_b(min(st + 1, nst - 1), bnx, snx);
        const int subs = 2 * st + 1 < kblocks ? 2 : 1;
#pragma unroll
        for (int s = 0; s < 2; s++) {
            if (s >= subs)
                break;
#pragma unroll
            for (int f = 0; f < NMF; f++) {
                const u32x4_t a = lds.codes[cur][f][rh][rl * 8 + ((4 * s + q) ^ rl)];
                const uint32_t sa = (lds.scales[cur][f][16 * s + ar] >> (8 * q)) & 0xFFu;
#pragma unroll
                for (int nf = 0; nf < A4_NF; nf++)
                    acc[f][nf] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        fp4_operand8(bcur[s][nf]), fp4_operand8(a), acc[f][nf], 4, 4, 0, (int)scur[s][nf], 0, (int)sa);
            }
        }
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
            for (int nf = 0; nf < A4_NF; nf++) {
                bcur[s][nf] = bnx[s][nf];
                scur[s][nf] = snx[s][nf];
            }
        // This wave's part of the next stage's A is in LDS and its reads of this stage's are done,
        // then the waves meet; the next stage's B prefetch (4 A4_NF loads, issued after the A
        // loads) stays in flight through the barrier and is waited for after it, so that no load
        // is outstanding at the loop head (the compiler does not order direct-to-LDS loads with
        // register loads in its wait counts, and a B load still pending there made it wait for the
        // next A stage before the multiplies).
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm_imm(4 * A4_NF));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("" ::: "memory");
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the last (repeated) A stage has landed before exit

    // GLU epilogue: fragments 2p (gate) and 2p + 1 (up) hold the same output columns.
    uint16_t *o = g.h;
    const int rbase = m0 + (lane & 15);
#pragma unroll
    for (int p = 0; p < A4_NF / 2; p++) {
        const int oc = n0 / 2 + p * 16 + 4 * q;
#pragma unroll
        for (int f = 0; f < NMF; f++) {
            const int r = rbase + f * 16;
            if (r >= m1)
                continue;
            float hf[4];
#pragma unroll
            for (int i = 0; i < 4; i++)
                hf[i] = silu_f32(acc[f][2 * p][i]) * acc[f][2 * p + 1][i];
            *reinterpret_cast<uint2 *>(o + (int64_t)r * g.ldh + oc) =
                make_uint2(pack_bf16x2(hf[0], hf[1]), pack_bf16x2(hf[2], hf[3]));
        }
    }
}

__global__ __launch_bounds__(WAVE * A4_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void a4_gateup_kernel(const A4GateupArgs g, int gx)
{
    __shared__ A4Lds lds;
    const int total = g.tiles[0] * gx;
    const int per = (total + A4_XCDS - 1) / A4_XCDS;
    const int slot = blockIdx.x / A4_XCDS;
    const int item = (blockIdx.x % A4_XCDS) * per + slot;
    if (slot >= per || item >= total)
        return;
    const int by = item / gx, bx = item % gx;
    const int4 t = reinterpret_cast<const int4 *>(g.tiles + TILE_HEADER_INTS)[by];
    // one code path per workgroup, chosen by the tile's row count
    const int nmf = __builtin_amdgcn_readfirstlane((t.z - t.y + 15) / 16);
    if (nmf <= 1)
        a4_tile<1>(g, bx, t.x, t.y, t.z, lds);
    else if (nmf == 2)
        a4_tile<2>(g, bx, t.x, t.y, t.z, lds);
    else if (nmf == 3)
        a4_tile<3>(g, bx, t.x, t.y, t.z, lds);
    else if (nmf == 4)
        a4_tile<4>(g, bx, t.x, t.y, t.z, lds);
    else if (nmf == 5)
        a4_tile<5>(g, bx, t.x, t.y, t.z, lds);
    else if (nmf == 6)
        a4_tile<6>(g, bx, t.x, t.y, t.z, lds);
    else
        a4_tile<8>(g, bx, t.x, t.y, t.z, lds);
}

hipError_t launch_a4_gateup(const A4GateupArgs &g, int max_tiles, hipStream_t st)
{
    if (!g.tiles || !g.zq || !g.zs || !g.B || !g.h || g.N <= 0 || g.N % A4_BN || g.K < MX_STEP || g.K % MX_STEP ||
        g.ldh < g.N / 2 || g.ldh % 4 || reinterpret_cast<uintptr_t>(g.zq) % 16 ||
        reinterpret_cast<uintptr_t>(g.zs) % 4 || reinterpret_cast<uintptr_t>(g.h) % 8)
        return hipErrorInvalidValue;
    if (max_tiles <= 0)
        return hipSuccess;
    const int gx = g.N / A4_BN;
    const int64_t grid = ((int64_t)gx * max_tiles + A4_XCDS - 1) / A4_XCDS * A4_XCDS;
    if (grid > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(a4_gateup_kernel, dim3((unsigned)grid), dim3(WAVE * A4_WAVES), 0, st, g, gx);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Grouped A4W4 gate|up product with the GLU for expert tiles of at most 16 rows (few tokens per
// expert), where the time is the HBM stream of the weights: the structure of the BF16 few-row
// kernel on the scaled FP4 x FP4 instruction. Workgroup (x, y) computes tile y of the list for the
// 64 columns 64 x .. 64 x + 63 (four 16-row weight blocks: gate, up, gate, up). Its WK waves split
// the K axis in whole MX blocks; a wave loads SB blocks' weights (codes and scales) and z (codes and
// the scale byte of its slice) before it multiplies them. The partial tiles are summed in LDS in
// wave order, then the GLU is written. Lane (q, c) of a fragment holds token row c (clamped to a
// valid row, never stored past the tile) and columns 4 q .. 4 q + 3.
template <int WK, int SB>
__global__ __launch_bounds__(WAVE *WK) void a4_small_kernel(const A4GateupArgs g)
{
    constexpr int BN = 64;
    __shared__ float red[WK * 16 * BN];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = threadIdx.x / WAVE;
    if ((int)blockIdx.y >= g.tiles[0])
        return;
    const int4 t = reinterpret_cast<const int4 *>(g.tiles + TILE_HEADER_INTS)[blockIdx.y];
    const int m0 = t.y, m1 = t.z;
    const int n0 = blockIdx.x * BN;
    const int kblocks = g.K / MX_STEP;
    const int s0 = (wv * kblocks) / WK, s1 = ((wv + 1) * kblocks) / WK;
    const int c = lane & 15, q = lane >> 4;
    const int r = min(m0 + c, m1 - 1);
    const int64_t row = g.a_index ? (int64_t)(g.a_index[r] / g.a_div) : (int64_t)r;
    const uint8_t *zrow = g.zq + row * (g.K / 2) + 16 * q;
    const uint8_t *srow = g.zs + row * (g.K / 32) + q;
    const uint8_t *Bg = g.B + (int64_t)t.x * g.b_stride;

    f32x4_t acc[4];
#pragma unroll
    for (int nf = 0; nf < 4; nf++)
        acc[nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s = s0; s < s1; s += SB) {
        u32x4_t bc[SB][4], a[SB];
        uint32_t bs[SB][4], as[SB];
#pragma unroll
        for (int u = 0; u < SB; u++) {
            const int kb = min(s + u, s1 - 1);   // past the wave's range: re-read (not multiplied)
#pragma unroll
            for (int nf = 0; nf < 4; nf++) {
                const uint8_t *p = Bg + ((int64_t)(n0 / 16 + nf) * kblocks + kb) * MX_BLOCK_BYTES;
                bc[u][nf] = load16_nt(p + lane * 16);
                bs[u][nf] = p[MX_CODE_BYTES + lane];
            }
            a[u] = load16(zrow + kb * (MX_STEP / 2));
            as[u] = srow[kb * 4];
        }
#pragma unroll
        for (int u = 0; u < SB; u++)
            if (s + u < s1)
#pragma unroll
                for (int nf = 0; nf < 4; nf++)
                    acc[nf] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        fp4_operand8(bc[u][nf]), fp4_operand8(a[u]), acc[nf], 4, 4, 0, (int)bs[u][nf], 0, (int)as[u]);
    }
#pragma unroll
    for (int nf = 0; nf < 4; nf++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            red[(wv * 16 + c) * BN + nf * 16 + 4 * q + i] = acc[nf][i];
    __syncthreads();
    // GLU: output column oc of this block pairs gate column 32 (oc / 16) + oc % 16 with the up
    // column 16 after it
    constexpr int BO = BN / 2;
    for (int idx = threadIdx.x; idx < 16 * BO; idx += WAVE * WK) {
        const int rr = idx / BO, oc = idx % BO;
        const int orow = m0 + rr;
        if (orow >= m1)
            continue;
        const int gc = (oc / 16) * 32 + (oc % 16), uc = gc + 16;
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int w = 0; w < WK; w++) {
            gs += red[(w * 16 + rr) * BN + gc];
            us += red[(w * 16 + rr) * BN + uc];
        }
        g.h[(int64_t)orow * g.ldh + n0 / 2 + oc] = (uint16_t)f32_to_bf16_bits(silu_f32(gs) * us);
    }
}

#ifndef A4_SMALL_SB
#define A4_SMALL_SB 1
#endif
hipError_t launch_a4_gateup_small(const A4GateupArgs &g, int max_tiles, hipStream_t st)
{
    if (!g.tiles || !g.zq || !g.zs || !g.B || !g.h || g.N <= 0 || g.N % 64 || g.K < MX_STEP || g.K % MX_STEP ||
        g.ldh < g.N / 2 || reinterpret_cast<uintptr_t>(g.zq) % 16)
        return hipErrorInvalidValue;
    if (max_tiles <= 0)
        return hipSuccess;
    if (max_tiles > 65535)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((a4_small_kernel<4, A4_SMALL_SB>), dim3(g.N / 64, max_tiles), dim3(WAVE * 4), 0, st, g);
    return hipGetLastError();
}

} // namespace mxmoe
