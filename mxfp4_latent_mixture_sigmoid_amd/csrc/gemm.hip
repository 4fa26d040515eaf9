// gemm.hip -- grouped MXFP4 expert products for few rows per expert (decode), where the time is
// the HBM stream of the expert weights.
//
// A is a row-major BF16 activation matrix, gathered row by row through the expert-sorted order; B
// is an expert's packed MXFP4 matrix (see common.hpp) streamed from HBM in fragment order so that
// every 16-byte lane load holds four matrix-core operands and a wave's load covers 1 KiB of
// contiguous memory. MXFP4 codes are converted to BF16 in registers with their E8M0 scale (gfx950's
// scaled FP4 conversion) right before the 16x16x32 BF16 instruction; accumulation is FP32. The
// waves of a workgroup split the K axis; their partial tiles are summed in LDS in a fixed order, so
// the result does not depend on timing. The epilogue writes BF16, or the GLU
// h = bf16(silu(gate) * up) from gate/up column pairs.
#include "kernels.hpp"

namespace mxmoe {

template <int MT, int NT, int WK>
__global__ __launch_bounds__(WAVE *WK) void gemm_kernel(const GemmArgs g)
{
    constexpr int BM = 16 * MT, BN = 16 * NT;
    constexpr int STEP = MX_STEP;
    __shared__ float red[WK * BM * BN];

    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = threadIdx.x / WAVE;

    // Column block fastest in the launch order: neighbouring workgroups stream neighbouring weights.
    if ((int)blockIdx.y >= g.tiles[0])
        return;
    const int4 t = reinterpret_cast<const int4 *>(g.tiles + TILE_HEADER_INTS)[blockIdx.y];
    const int group = t.x, m0 = t.y, m1 = t.z;
    const int n0 = blockIdx.x * BN;

    // Activation rows of this lane for each 16-row fragment (gathered when a_index is set).
    const uint16_t *arow[MT];
    bool aval[MT];
#pragma unroll
    for (int mf = 0; mf < MT; mf++) {
        const int r = m0 + mf * 16 + (lane & 15);
        aval[mf] = r < m1;
        int64_t row = 0;
        if (aval[mf])
            row = g.a_index ? (int64_t)(g.a_index[r] / g.a_div) : (int64_t)r;
        arow[mf] = g.A + row * g.lda + 8 * (lane >> 4);
    }

    const int nsteps = g.K / STEP;
    const int s0 = (wv * nsteps) / WK, s1 = ((wv + 1) * nsteps) / WK;
    const uint8_t *Bg = g.B + (int64_t)group * g.b_stride;

    f32x4_t acc[MT][NT];
#pragma unroll
    for (int mf = 0; mf < MT; mf++)
#pragma unroll
        for (int nf = 0; nf < NT; nf++)
            acc[mf][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const u32x4_t zero4 = {0u, 0u, 0u, 0u};
    {
        for (int s = s0; s < s1; s++) {
            u32x4_t codes[NT];
            uint32_t sc[NT];
#pragma unroll
            for (int nf = 0; nf < NT; nf++) {
                const uint8_t *blk = Bg + ((int64_t)(n0 / 16 + nf) * nsteps + s) * MX_BLOCK_BYTES;
                codes[nf] = load16_nt(blk + lane * 16);
                sc[nf] = load4_nt(blk + MX_CODE_BYTES + 4 * (lane & 15));
            }
            u32x4_t a[MT][4];
#pragma unroll
            for (int mf = 0; mf < MT; mf++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    a[mf][j] = aval[mf] ? load16(arow[mf] + s * STEP + 32 * j) : zero4;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                bf16x8_t b[NT];
#pragma unroll
                for (int nf = 0; nf < NT; nf++)
                    b[nf] = mx_dequant8(codes[nf][j], e8m0_to_f32((sc[nf] >> (8 * j)) & 0xFFu));
#pragma unroll
                for (int mf = 0; mf < MT; mf++)
#pragma unroll
                    for (int nf = 0; nf < NT; nf++)
                        acc[mf][nf] = mfma16(as_bf16x8(a[mf][j]), b[nf], acc[mf][nf]);
            }
        }
    }

    // Partial tiles to LDS: lane l holds rows 4 (l/16) + i, column l % 16 of each fragment.
#pragma unroll
    for (int mf = 0; mf < MT; mf++)
#pragma unroll
        for (int nf = 0; nf < NT; nf++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int row = mf * 16 + 4 * (lane >> 4) + i, col = nf * 16 + (lane & 15);
                red[(wv * BM + row) * BN + col] = acc[mf][nf][i];
            }
    __syncthreads();

    const OutDesc d = g.lo;
    const int nthr = WAVE * WK;
    if (d.kind == OUT_GLU) {
        // Column pairs: within each 32 columns, 16 gate columns then the 16 matching up columns.
        constexpr int BO = BN / 2;
        for (int idx = threadIdx.x; idx < BM * BO; idx += nthr) {
            const int row = idx / BO, oc = idx % BO;
            const int r = m0 + row;
            if (r >= m1)
                continue;
            const int gc = (oc / 16) * 32 + (oc % 16), uc = gc + 16;
            float gs = 0.f, us = 0.f;
#pragma unroll
            for (int w = 0; w < WK; w++) {
                gs += red[(w * BM + row) * BN + gc];
                us += red[(w * BM + row) * BN + uc];
            }
            const float h = silu_f32(gs) * us;
            uint16_t *o = reinterpret_cast<uint16_t *>(d.ptr);
            o[(int64_t)r * d.ld + (n0 - d.col0) / 2 + oc] = (uint16_t)f32_to_bf16_bits(h);
        }
    } else {
        for (int idx = threadIdx.x; idx < BM * BN; idx += nthr) {
            const int row = idx / BN, col = idx % BN;
            const int r = m0 + row, n = n0 + col;
            if (r >= m1 || n >= d.n_valid)
                continue;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < WK; w++)
                v += red[(w * BM + row) * BN + col];
            reinterpret_cast<uint16_t *>(d.ptr)[(int64_t)r * d.ld + (n - d.col0)] = (uint16_t)f32_to_bf16_bits(v);
        }
    }
}

// Grouped MXFP4 product for expert tiles of at most 16 rows (few tokens per expert), where the
// time is the HBM stream of the expert weights. Each wave owns NT 16-row blocks of B and a K range
// of whole 128-input blocks; for up to MAXS blocks at a time it issues every code, scale and
// activation load first (addresses clamped into its range, so no load is conditional) and only
// then converts and multiplies, so a wave keeps MAXS x NT KiB of weights in flight. WN waves
// split the columns, WK waves the K range (summed in LDS in a fixed order).
template <int NT, int WN, int WK, int MAXS>
__global__ __launch_bounds__(WAVE *WN *WK) void mx_stream_kernel(const GemmArgs g)
{
    constexpr int BN = 16 * NT * WN;
    __shared__ float red[WK * 16 * BN];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = threadIdx.x / WAVE, wn = wv % WN, wk = wv / WN;

    if ((int)blockIdx.y >= g.tiles[0])
        return;
    const int4 tile = reinterpret_cast<const int4 *>(g.tiles + TILE_HEADER_INTS)[blockIdx.y];
    const int group = tile.x, m0 = tile.y, m1 = tile.z;
    const int n0 = blockIdx.x * BN;

    const int r = m0 + (lane & 15);
    const bool aval = r < m1;
    int64_t arow_idx = 0;
    if (aval)
        arow_idx = g.a_index ? (int64_t)(g.a_index[r] / g.a_div) : (int64_t)r;
    const uint16_t *arow = g.A + arow_idx * g.lda + 8 * (lane >> 4);

    const int nblk = g.K / MX_STEP;
    const int kb0 = (wk * nblk) / WK, kb1 = ((wk + 1) * nblk) / WK;
    const uint8_t *Bg = g.B + (int64_t)group * g.b_stride;
    const int nb0 = n0 / 16 + wn * NT;
    const bool wact = nb0 + NT <= g.N / 16;          // waves past the last column block idle

    f32x4_t acc[NT];
#pragma unroll
    for (int nf = 0; nf < NT; nf++)
        acc[nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const u32x4_t zero4 = {0u, 0u, 0u, 0u};

    for (int kb = kb0; wact && kb < kb1; kb += MAXS) {
        const int cnt = min(MAXS, kb1 - kb);
        u32x4_t codes[MAXS][NT];
        uint32_t sc[MAXS][NT];
        u32x4_t a[MAXS][4];
#pragma unroll
        for (int s = 0; s < MAXS; s++) {
            const int blk = kb + min(s, cnt - 1);
#pragma unroll
            for (int nf = 0; nf < NT; nf++) {
                const uint8_t *p = Bg + ((int64_t)(nb0 + nf) * nblk + blk) * MX_BLOCK_BYTES;
                codes[s][nf] = load16_nt(p + lane * 16);
                sc[s][nf] = load4_nt(p + MX_CODE_BYTES + 4 * (lane & 15));
            }
        }
#pragma unroll
        for (int s = 0; s < MAXS; s++) {
            const int blk = kb + min(s, cnt - 1);
#pragma unroll
            for (int j = 0; j < 4; j++)
                a[s][j] = aval ? load16(arow + blk * MX_STEP + 32 * j) : zero4;
        }
#pragma unroll
        for (int s = 0; s < MAXS; s++) {
            if (s < cnt) {
#pragma unroll
                for (int j = 0; j < 4; j++)
#pragma unroll
                    for (int nf = 0; nf < NT; nf++)
                        acc[nf] = mfma16(as_bf16x8(a[s][j]),
                                         mx_dequant8(codes[s][nf][j], e8m0_to_f32((sc[s][nf] >> (8 * j)) & 0xFFu)),
                                         acc[nf]);
            }
        }
    }

#pragma unroll
    for (int nf = 0; nf < NT; nf++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int row = 4 * (lane >> 4) + i, col = (wn * NT + nf) * 16 + (lane & 15);
            red[(wk * 16 + row) * BN + col] = acc[nf][i];
        }
    __syncthreads();

    const OutDesc d = g.lo;
    const int nthr = WAVE * WN * WK;
    if (d.kind == OUT_GLU) {
        constexpr int BO = BN / 2;
        for (int idx = threadIdx.x; idx < 16 * BO; idx += nthr) {
            const int row = idx / BO, oc = idx % BO;
            const int rr = m0 + row;
            if (rr >= m1)
                continue;
            const int gc = (oc / 16) * 32 + (oc % 16), uc = gc + 16;
            float gs = 0.f, us = 0.f;
#pragma unroll
            for (int w = 0; w < WK; w++) {
                gs += red[(w * 16 + row) * BN + gc];
                us += red[(w * 16 + row) * BN + uc];
            }
            reinterpret_cast<uint16_t *>(d.ptr)[(int64_t)rr * d.ld + (n0 - d.col0) / 2 + oc] =
                (uint16_t)f32_to_bf16_bits(silu_f32(gs) * us);
        }
    } else {
        for (int idx = threadIdx.x; idx < 16 * BN; idx += nthr) {
            const int row = idx / BN, col = idx % BN;
            const int rr = m0 + row, n = n0 + col;
            if (rr >= m1 || n >= d.n_valid)
                continue;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < WK; w++)
                v += red[(w * 16 + row) * BN + col];
            reinterpret_cast<uint16_t *>(d.ptr)[(int64_t)rr * d.ld + (n - d.col0)] = (uint16_t)f32_to_bf16_bits(v);
        }
    }
}

template <int NT, int WN, int WK, int MAXS>
static hipError_t launch_stream(const GemmArgs &g, int max_tiles, hipStream_t st)
{
    constexpr int BN = 16 * NT * WN;
    if (g.N % (16 * NT) != 0 || g.K % MX_STEP != 0 || !g.tiles)
        return hipErrorInvalidValue;
    if (max_tiles <= 0)
        return hipSuccess;
    if (max_tiles > 65535)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((mx_stream_kernel<NT, WN, WK, MAXS>), dim3((g.N + BN - 1) / BN, max_tiles),
                       dim3(WAVE * WN * WK), 0, st, g);
    return hipGetLastError();
}

template <int MT, int NT, int WK>
static hipError_t launch(const GemmArgs &g, int grid_m, hipStream_t st)
{
    constexpr int BN = 16 * NT;
    if (g.N % BN != 0 || g.K % MX_STEP != 0 || !g.tiles || g.lo.kind == OUT_F32 || g.split < g.N)
        return hipErrorInvalidValue;
    if (grid_m <= 0)
        return hipSuccess;
    if (grid_m > 65535)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_kernel<MT, NT, WK>), dim3(g.N / BN, grid_m), dim3(WAVE * WK), 0, st, g);
    return hipGetLastError();
}

// Grouped MXFP4 products over the tile list (upper bound `max_tiles` workgroup rows).
hipError_t launch_gemm_grouped(const GemmArgs &g, GemmShape shape, int max_tiles, hipStream_t st)
{
    switch (shape) {
    case GEMM_MX_GLU_M16:
        return launch<1, 2, 4>(g, max_tiles, st);
    case GEMM_MX_M16_N64:
        return launch_stream<4, 1, 1, 3>(g, max_tiles, st);
    case GEMM_MX_GLU_M16_N64:
        return launch<1, 4, 4>(g, max_tiles, st);
    default:
        return hipErrorInvalidValue;
    }
}

} // namespace mxmoe
