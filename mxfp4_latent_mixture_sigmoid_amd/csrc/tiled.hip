// tiled.hip -- matrix-core GEMM for many tokens, C = A . B^T, where the time is BF16 MFMA work.
//
// Each of the four waves of a workgroup owns a 128 x 64 output tile (8 x 4 fragments of the
// 16x16x32 BF16 instruction, 128 FP32 accumulators per lane), small enough for two waves per SIMD;
// at the matrix-core peak this reads ~64 B/clk/CU from LDS and ~32 B/clk/CU from cache. The
// workgroup is 1 x 4 waves (128 rows x 256 columns) or 2 x 2 waves (256 x 128).
//  * A (activations, optionally gathered rows) is staged per 128-wide K stage into LDS in operand
//    order -- for K sub-step s and 16-row fragment f, one 1 KiB block holding lane l's operand at
//    slot l -- so the writes and the reads are sequential (no bank conflicts). Two LDS buffers
//    alternate: stage k+1 is loaded into registers while stage k is multiplied, then written.
//  * B (weights) is read straight from the packed fragment layout into registers, one K
//    sub-step (BF16) or one 128-wide MX block (MXFP4) ahead of its use; MXFP4 codes are
//    converted to BF16 with their E8M0 scale right before the multiply.
// Rows past the tile end read a clamped valid row and are never stored; column blocks past N are
// skipped by whole waves; K needs only be a multiple of 32 (BF16) or 128 (MXFP4).
#include "kernels.hpp"

namespace mxmoe {

constexpr int TL_WAVE_M = 128, TL_WAVE_N = 64;
constexpr int TL_MF = TL_WAVE_M / 16, TL_NF = TL_WAVE_N / 16;   // 8 x 4 fragments per wave
constexpr int TL_STAGE_K = 128;                                 // K per LDS stage
constexpr int TL_SUB = TL_STAGE_K / 32;                         // 32-wide sub-steps per stage

template <int WM, int WN, bool MX>
__global__ __launch_bounds__(WAVE * 4) void tiled_kernel(const GemmArgs g)
{
    static_assert(WM * WN == 4, "four waves");
    constexpr int BM = TL_WAVE_M * WM, BN = TL_WAVE_N * WN;
    constexpr int MFW = BM / 16;                                // 16-row fragments per workgroup
    constexpr int SLOTS = TL_SUB * MFW * WAVE;                  // 16-byte slots per stage
    constexpr int PER_THREAD = SLOTS / (WAVE * 4);
    __shared__ u32x4_t lds[2][SLOTS];

    const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
    const int wm = wv / WN, wn = wv % WN;

    int group = 0, m0, m1;
    if (g.tiles) {
        if ((int)blockIdx.y >= g.tiles[0])
            return;
        const int4 t = reinterpret_cast<const int4 *>(g.tiles + TILE_HEADER_INTS)[blockIdx.y];
        group = t.x;
        m0 = t.y;
        m1 = t.z;
    } else {
        m0 = blockIdx.y * BM;
        m1 = min(g.M, m0 + BM);
    }
    const int n0 = blockIdx.x * BN + wn * TL_WAVE_N;            // this wave's first column
    const int nblocks = g.N / 16;
    const uint8_t *Bg = g.B + (int64_t)group * g.b_stride;

    // ---- A staging. Thread t fills slots t + 256 u: its lane slot (t % 64) is fixed, so its row
    // within a fragment (t % 16) and its K quarter ((t % 64) / 16) are too; block t / 64 + 4 u runs
    // over fragments f = wv + 4 (u % FR) (FR = MFW / 4 distinct rows) and sub-steps s = u / FR.
    constexpr int FR = MFW / 4;
    const uint16_t *arow[FR];
#pragma unroll
    for (int i = 0; i < FR; i++) {
        const int r = min(m0 + (wv + 4 * i) * 16 + (lane & 15), m1 - 1);   // clamped valid row
        const int64_t row = g.a_index ? (int64_t)(g.a_index[r] / g.a_div) : (int64_t)r;
        arow[i] = g.A + row * g.lda + 8 * (lane >> 4);
    }
    const int nstages = (g.K + TL_STAGE_K - 1) / TL_STAGE_K;
    auto load_a = [&](int stage, u32x4_t *v) {
#pragma unroll
        for (int u = 0; u < PER_THREAD; u++) {
            const int k = min(stage * TL_STAGE_K + (u / FR) * 32, g.K - 32);
            v[u] = load16(arow[u % FR] + k);
        }
    };
    auto store_a = [&](int buf, const u32x4_t *v) {
#pragma unroll
        for (int u = 0; u < PER_THREAD; u++)
            lds[buf][threadIdx.x + u * WAVE * 4] = v[u];
    };

    // ---- B fragments of this wave
    bool nval[TL_NF];
#pragma unroll
    for (int nf = 0; nf < TL_NF; nf++)
        nval[nf] = (n0 / 16 + nf) < nblocks;

    f32x4_t acc[TL_MF][TL_NF];
#pragma unroll
    for (int i = 0; i < TL_MF; i++)
#pragma unroll
        for (int j = 0; j < TL_NF; j++)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    {
        u32x4_t av[PER_THREAD];
        load_a(0, av);
        store_a(0, av);
    }
    __syncthreads();

    const bool wave_active = n0 < g.N;
    for (int st = 0; st < nstages; st++) {
        const int cur = st & 1;
        u32x4_t an[PER_THREAD];
        if (st + 1 < nstages)
            load_a(st + 1, an);

        if (wave_active) {
            if constexpr (MX) {
                const int kb = st;                               // one MX block per stage
                u32x4_t codes[TL_NF];
                uint32_t sc[TL_NF];
#pragma unroll
                for (int nf = 0; nf < TL_NF; nf++) {
                    const int nb = min(n0 / 16 + nf, nblocks - 1);
                    const uint8_t *p = Bg + ((int64_t)nb * (g.K / MX_STEP) + kb) * MX_BLOCK_BYTES;
                    codes[nf] = load16_nt(p + lane * 16);
                    sc[nf] = load4_nt(p + MX_CODE_BYTES + 4 * (lane & 15));
                }
#pragma unroll
                for (int s = 0; s < TL_SUB; s++) {
                    u32x4_t a[TL_MF];
#pragma unroll
                    for (int f = 0; f < TL_MF; f++)
                        a[f] = lds[cur][(s * MFW + wm * TL_MF + f) * WAVE + lane];
#pragma unroll
                    for (int nf = 0; nf < TL_NF; nf++) {
                        if (!nval[nf])
                            continue;
                        const bf16x8_t b = mx_dequant8(codes[nf][s], e8m0_to_f32((sc[nf] >> (8 * s)) & 0xFFu));
#pragma unroll
                        for (int f = 0; f < TL_MF; f++)
                            acc[f][nf] = mfma16(as_bf16x8(a[f]), b, acc[f][nf]);
                    }
                }
            } else {
                const int ks = g.K / BF16_STEP;
                u32x4_t bcur[TL_NF], bnext[TL_NF];
                auto load_b = [&](int kstep, u32x4_t *b) {
#pragma unroll
                    for (int nf = 0; nf < TL_NF; nf++) {
                        const int nb = min(n0 / 16 + nf, nblocks - 1);
                        b[nf] = load16_nt(Bg + bf16_block_index(nb, min(kstep, ks - 1), g.N, g.K) * BF16_BLOCK_BYTES +
                                          lane * 16);
                    }
                };
                load_b(st * TL_SUB, bcur);
#pragma unroll
                for (int s = 0; s < TL_SUB; s++) {
                    const int kstep = st * TL_SUB + s;
                    if (s + 1 < TL_SUB)
                        load_b(kstep + 1, bnext);
                    if (kstep < ks) {
                        u32x4_t a[TL_MF];
#pragma unroll
                        for (int f = 0; f < TL_MF; f++)
                            a[f] = lds[cur][(s * MFW + wm * TL_MF + f) * WAVE + lane];
#pragma unroll
                        for (int nf = 0; nf < TL_NF; nf++) {
                            if (!nval[nf])
                                continue;
#pragma unroll
                            for (int f = 0; f < TL_MF; f++)
                                acc[f][nf] = mfma16(as_bf16x8(a[f]), as_bf16x8(bcur[nf]), acc[f][nf]);
                        }
                    }
#pragma unroll
                    for (int nf = 0; nf < TL_NF; nf++)
                        bcur[nf] = bnext[nf];
                }
            }
        }
        if (st + 1 < nstages) {
            store_a(cur ^ 1, an);
            __syncthreads();
        }
    }

    if (!wave_active)
        return;
    // ---- epilogue: lane holds rows 4(l/16)+i of each fragment, column l % 16
    const OutDesc d = (n0 < g.split) ? g.lo : g.hi;
    const int rbase = m0 + wm * TL_WAVE_M + 4 * (lane >> 4);
    if (d.kind == OUT_GLU) {
        // fragments 2p (gate) and 2p+1 (up) hold the same 16 output columns
        uint16_t *o = reinterpret_cast<uint16_t *>(d.ptr);
#pragma unroll
        for (int p = 0; p < TL_NF / 2; p++) {
            if (!nval[2 * p + 1])
                continue;
            const int oc = (n0 - d.col0) / 2 + p * 16 + (lane & 15);
#pragma unroll
            for (int f = 0; f < TL_MF; f++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int r = rbase + f * 16 + i;
                    if (r < m1)
                        o[(int64_t)r * d.ld + oc] =
                            (uint16_t)f32_to_bf16_bits(silu_f32(acc[f][2 * p][i]) * acc[f][2 * p + 1][i]);
                }
        }
    } else {
#pragma unroll
        for (int nf = 0; nf < TL_NF; nf++) {
            const int n = n0 + nf * 16 + (lane & 15);
            if (!nval[nf] || n >= d.n_valid)
                continue;
            const float bias = (d.kind == OUT_F32 && d.bias) ? d.bias[n] : 0.f;
#pragma unroll
            for (int f = 0; f < TL_MF; f++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int r = rbase + f * 16 + i;
                    if (r >= m1)
                        continue;
                    if (d.kind == OUT_F32)
                        reinterpret_cast<float *>(d.ptr)[(int64_t)r * d.ld + (n - d.col0)] = acc[f][nf][i] + bias;
                    else
                        reinterpret_cast<uint16_t *>(d.ptr)[(int64_t)r * d.ld + (n - d.col0)] =
                            (uint16_t)f32_to_bf16_bits(acc[f][nf][i]);
                }
        }
    }
}

template <int WM, int WN, bool MX>
static hipError_t launch_tiled_t(const GemmArgs &g, int grid_m, hipStream_t st)
{
    constexpr int BN = TL_WAVE_N * WN;
    if (g.N % 16 || g.K % (MX ? MX_STEP : BF16_STEP) || g.K < 8)
        return hipErrorInvalidValue;
    if (grid_m <= 0)
        return hipSuccess;
    if (grid_m > 65535)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((tiled_kernel<WM, WN, MX>), dim3((g.N + BN - 1) / BN, grid_m), dim3(WAVE * 4), 0, st, g);
    return hipGetLastError();
}

int tiled_rows(TiledShape shape) { return shape == TILED_256x256 ? 256 : 128; }

hipError_t launch_tiled(const GemmArgs &g, TiledShape shape, bool mx, int max_tiles, hipStream_t st)
{
    const int bm = tiled_rows(shape);
    const int grid_m = g.tiles ? max_tiles : (g.M + bm - 1) / bm;
    if (shape == TILED_128x512)
        return mx ? launch_tiled_t<1, 4, true>(g, grid_m, st) : launch_tiled_t<1, 4, false>(g, grid_m, st);
    if (shape == TILED_256x256)
        return mx ? launch_tiled_t<2, 2, true>(g, grid_m, st) : launch_tiled_t<2, 2, false>(g, grid_m, st);
    return hipErrorInvalidValue;
}

} // namespace mxmoe
