// tiled.hip -- matrix-core GEMM for many tokens, C = A . B^T, where the time is BF16 MFMA work.
//
// Each of the four waves of a workgroup owns a 128 x 64 output tile (8 x 4 fragments of the
// 16x16x32 BF16 instruction, 128 FP32 accumulators per lane); the workgroup covers 128 rows x 256
// columns. At the matrix-core peak this reads ~64 B/clk/CU from LDS and ~47 B/clk/CU (BF16 B) or
// ~25 B/clk/CU (MXFP4 B) from cache.
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

#include <algorithm>

namespace mxmoe {

constexpr int TL_WAVE_M = 128, TL_WAVE_N = 64;
constexpr int TL_NF = TL_WAVE_N / 16;   // 16-column fragments per wave (and TL_WAVE_M / 16 = 8 row fragments)
constexpr int TL_STAGE_K = 128;                                 // K per LDS stage
constexpr int TL_SUB = TL_STAGE_K / 32;                         // 32-wide sub-steps per stage


constexpr int TL_XCDS = 8;      // workgroups are dealt to the XCDs round-robin by linear id
constexpr int TL_GROUP_M = 8;   // dense products: M tiles per group, walked M-fastest

// Linear workgroup id -> (N tile, M tile or tile-list entry), XCD-major: XCD c takes the contiguous
// run c*per .. c*per+per-1 of the work items, so the workgroups sharing one L2 also share operands.
// Tile lists: items run tile-major (the N tiles of one tile, then the next tile of the same
// expert). Dense: groups of TL_GROUP_M M tiles, M-fastest within a group. False past the end.
__device__ inline bool tiled_item(const GemmArgs &g, int gx, int gy, int &bx, int &by)
{
    const int total = g.tiles ? g.tiles[0] * gx : gx * gy;
    const int per = (total + TL_XCDS - 1) / TL_XCDS;
    const int slot = blockIdx.x / TL_XCDS;
    const int item = (blockIdx.x % TL_XCDS) * per + slot;
    if (slot >= per || item >= total)
        return false;
    if (g.tiles) {
        by = item / gx;
        bx = item % gx;
    } else {
        const int first = item / (TL_GROUP_M * gx) * TL_GROUP_M;
        const int rows = min(gy - first, TL_GROUP_M);
        const int in = item - first * gx;
        by = first + in % rows;
        bx = in / rows;
    }
    return true;
}

constexpr int TL_BM = TL_WAVE_M, TL_BN = TL_WAVE_N * 4;   // four waves side by side along N
constexpr int TL_MFW = TL_BM / 16;                         // 16-row fragments per workgroup
constexpr int TL_SLOTS = TL_SUB * TL_MFW * WAVE;           // 16-byte A slots per stage

// One 128 x 256 output tile (rows m0 .. m1-1 valid) of which only the first NMF 16-row fragments
// hold valid rows: the A staging, the MFMAs and the stores cover those fragments only, so a short
// tile (an expert's last rows) costs in proportion to its rows plus its B stream.
template <bool MX, int NMF>
__device__ __attribute__((always_inline)) inline void tiled_tile(const GemmArgs &g, int bx, int group, int m0, int m1,
                                                                 u32x4_t (*lds)[TL_SLOTS])
{
    static_assert(NMF >= 2 && NMF <= 8 && NMF != 7, "row fragments per tile");
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);   // wave-uniform
    const int n0 = bx * TL_BN + wv * TL_WAVE_N;                  // this wave's first column
    const int nblocks = g.N / 16;
    const uint8_t *Bg = g.B + (int64_t)group * g.b_stride;

    // ---- A staging. A stage holds TL_SUB x NMF 1 KiB blocks (sub-step s, fragment f at block
    // s * TL_MFW + f; slot 4 r + (c ^ chunk_swizzle(r)) holds row f*16 + r, inputs s*32 + 8c .. +7, so the
    // loads of slots 4r .. 4r+3 -- four consecutive lanes -- share a row). Thread t fills lane slot
    // t % 64 of blocks b = wv + 4u (u < NMF), b -> (s, f) = (b / NMF, b % NMF): its fragment row
    // f = (wv + 4u) % NMF repeats with period FR = NMF / gcd(NMF, 4) in u (NMF = 2..6, 8: 1, 3, 1,
    // 5, 3, 2 distinct rows), so row pointer u % FR serves load u.
    constexpr int FR = NMF / (NMF % 4 == 0 ? 4 : NMF % 2 == 0 ? 2 : 1);
    const uint16_t *arow[FR];
#pragma unroll
    for (int i = 0; i < FR; i++) {
        const int f = (wv + 4 * i) % NMF;
        const int r = min(m0 + f * 16 + (lane >> 2), m1 - 1);   // clamped valid row
        const int64_t row = g.a_index ? (int64_t)(g.a_index[r] / g.a_div) : (int64_t)r;
        arow[i] = g.A + row * g.lda + 8 * ((lane & 3) ^ chunk_swizzle(lane >> 2));
    }
    const int nstages = (g.K + TL_STAGE_K - 1) / TL_STAGE_K;
    auto load_a = [&](int stage, u32x4_t *v) {
#pragma unroll
        for (int u = 0; u < NMF; u++) {
            const int sub = (wv + 4 * u) / NMF;
            const int k = min(stage * TL_STAGE_K + sub * 32, g.K - 32);
            v[u] = load16(arow[u % FR] + k);
        }
    };
    auto store_a = [&](int buf, const u32x4_t *v) {
#pragma unroll
        for (int u = 0; u < NMF; u++) {
            const int b = wv + 4 * u;
            lds[buf][((b / NMF) * TL_MFW + b % NMF) * WAVE + lane] = v[u];
        }
    };
    // MXFP4 products stage A by direct global->LDS loads instead, with no register round trip, and
    // as whole 128-byte lines: a stage is 16 rows x 256 bytes per fragment (4 KiB, row r at
    // 256 r), one wave instruction fills 4 rows of it (1 KiB: lane l takes row 4 q + l / 16 of
    // the fragment, where q is the wave, and position l % 16 of that row). Position p of row r holds
    // 16-byte chunk p ^ r, so that the operand reads -- rows 0..15 of one chunk -- fall in distinct
    // banks. (The operand-order alternative, 16 rows x 64 bytes per instruction, fetches half lines:
    // ~9 against ~25 TB/s from L2 in a streaming probe, and the line's other half is fetched again
    // by the next sub-step's instruction.) The compiler does not track these loads into LDS, so the
    // stage loop waits for them itself (vmcnt) before the barrier that publishes the stage.
    const uint16_t *aline[NMF];
#pragma unroll
    for (int u = 0; u < NMF; u++) {
        const int rf = wv * 4 + (lane >> 4);                        // row of fragment u
        const int r = min(m0 + u * 16 + rf, m1 - 1);                // clamped valid row
        const int64_t row = g.a_index ? (int64_t)(g.a_index[r] / g.a_div) : (int64_t)r;
        aline[u] = g.A + row * g.lda + 8 * ((lane & 15) ^ rf);
    }
    auto issue_a = [&](int stage, int buf) {
        const int k = min(stage, nstages - 1) * TL_STAGE_K;
#pragma unroll
        for (int u = 0; u < NMF; u++)
            __builtin_amdgcn_global_load_lds(aline[u] + k,
                                             (__attribute__((address_space(3))) void *)&lds[buf][(u * 4 + wv) * WAVE],
                                             16, 0, 0);
    };

    // ---- B fragments of this wave
    bool nval[TL_NF];
#pragma unroll
    for (int nf = 0; nf < TL_NF; nf++)
        nval[nf] = (n0 / 16 + nf) < nblocks;

    f32x4_t acc[NMF][TL_NF];
#pragma unroll
    for (int i = 0; i < NMF; i++)
#pragma unroll
        for (int j = 0; j < TL_NF; j++)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const bool wave_active = n0 < g.N;
    // B of this wave, prefetched ahead of use: MXFP4 one stage (128 inputs) ahead, BF16 one 32-wide
    // step ahead (across stage boundaries). Past-the-end prefetches re-read the last valid block.
    const int ks = g.K / BF16_STEP;
    const int kblk = g.K / MX_STEP;
    auto load_mx = [&](int stage, u32x4_t *codes, uint32_t *sc) {
#pragma unroll
        for (int nf = 0; nf < TL_NF; nf++) {
            const int nb = min(n0 / 16 + nf, nblocks - 1);
            const uint8_t *p = Bg + ((int64_t)nb * kblk + min(stage, kblk - 1)) * MX_BLOCK_BYTES;
            // cached loads: the row tiles of one expert re-read its weights (non-temporal loads,
            // which leave L2 first, made the product 3-6% slower)
            codes[nf] = load16(p + lane * 16);
            sc[nf] = *reinterpret_cast<const uint32_t *>(p + MX_CODE_BYTES + 4 * (lane & 15));
        }
    };
    auto load_b = [&](int kstep, u32x4_t *b) {
#pragma unroll
        for (int nf = 0; nf < TL_NF; nf++) {
            const int nb = min(n0 / 16 + nf, nblocks - 1);
            b[nf] = load16(Bg + bf16_block_index(nb, min(kstep, ks - 1), g.N, g.K) * BF16_BLOCK_BYTES + lane * 16);
        }
    };
    // The stage loop is one basic block: waves past N multiply clamped (valid) B and store nothing,
    // and the last stage re-stages a clamped valid A stage, so no value crosses a branch.
    u32x4_t bcur[TL_NF];
    uint32_t sccur[TL_NF];
    if constexpr (MX) {
        // The first stage's B is loaded before the first A stage, so the prologue's full wait
        // covers it: the compiler does not order direct-to-LDS loads with register loads in its
        // wait counts, and a B load still pending at the loop head made it wait for the whole
        // next A stage (vmcnt(0)) before every stage's multiplies.
        load_mx(0, bcur, sccur);
        issue_a(0, 0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    } else {
        u32x4_t av[NMF];
        load_a(0, av);
        store_a(0, av);
        __syncthreads();
        load_b(0, bcur);
    }

    for (int st = 0; st < nstages; st++) {
        const int cur = st & 1;
        u32x4_t an[MX ? 1 : NMF];
        if constexpr (MX)
            issue_a(min(st + 1, nstages - 1), cur ^ 1);   // before this stage's B prefetch (vmcnt order)
        else
            load_a(min(st + 1, nstages - 1), an);

        {
            if constexpr (MX) {
                u32x4_t bnx[TL_NF];
                uint32_t scnx[TL_NF];
                load_mx(st + 1, bnx, scnx);
#pragma unroll
                for (int s = 0; s < TL_SUB; s++) {
                    u32x4_t a[NMF];
                    const int ar = lane & 15, ac = ((s * 4 + (lane >> 4)) ^ ar);   // row, position of its chunk
#pragma unroll
                    for (int f = 0; f < NMF; f++)
                        a[f] = lds[cur][f * 256 + ar * 16 + ac];
#pragma unroll
                    for (int nf = 0; nf < TL_NF; nf++) {
                        const bf16x8_t b = mx_dequant8(bcur[nf][s], e8m0_to_f32((sccur[nf] >> (8 * s)) & 0xFFu));
#pragma unroll
                        for (int f = 0; f < NMF; f++)
                            acc[f][nf] = mfma16(b, as_bf16x8(a[f]), acc[f][nf]);
                    }
                    __builtin_amdgcn_sched_barrier(0);   // keep one sub-step's operands live at a time
                }
#pragma unroll
                for (int nf = 0; nf < TL_NF; nf++) {
                    bcur[nf] = bnx[nf];
                    sccur[nf] = scnx[nf];
                }
            } else {
#pragma unroll
                for (int s = 0; s < TL_SUB; s++) {
                    const int kstep = st * TL_SUB + s;
                    u32x4_t bnx[TL_NF];
                    load_b(kstep + 1, bnx);
                    if (kstep < ks) {
                        u32x4_t a[NMF];
#pragma unroll
                        for (int f = 0; f < NMF; f++)
                            a[f] = lds[cur][(s * TL_MFW + f) * WAVE + (lane & 15) * 4 + ((lane >> 4) ^ chunk_swizzle(lane & 15))];
#pragma unroll
                        for (int nf = 0; nf < TL_NF; nf++)
#pragma unroll
                            for (int f = 0; f < NMF; f++)
                                acc[f][nf] = mfma16(as_bf16x8(bcur[nf]), as_bf16x8(a[f]), acc[f][nf]);
                    }
#pragma unroll
                    for (int nf = 0; nf < TL_NF; nf++)
                        bcur[nf] = bnx[nf];
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        // This wave's part of the next stage's A is in LDS and its reads of this stage's are done,
        // then the waves meet. The wait leaves the next stage's B prefetch (issued after the A loads:
        // 2 TL_NF MXFP4 loads) in flight; a __syncthreads would wait for every outstanding global
        // load and expose that latency once per stage.
        asm volatile("" ::: "memory");
        if constexpr (MX) {
            __builtin_amdgcn_s_waitcnt(vmcnt_lgkm_imm(2 * TL_NF));
        } else {
            store_a(cur ^ 1, an);
            __builtin_amdgcn_s_waitcnt(LGKM_ZERO);
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
    if constexpr (MX)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the last (repeated) A stage has landed before exit

    if (!wave_active)
        return;
    // ---- epilogue. The weights are the first MFMA operand, so lane (q = l / 16, c = l % 16) of
    // fragment (f, nf) holds token row f*16 + c and the four consecutive columns nf*16 + 4q + i:
    // one 8-byte (BF16) or 16-byte (FP32) store per fragment when the output is aligned for it.
    const OutDesc d = out_region(g, n0);
    const int q = lane >> 4;
    const int rbase = m0 + (lane & 15);
    const bool vec = (d.ld % 4 == 0) && (d.col0 % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(d.ptr) % (d.kind == OUT_F32 ? 16 : 8) == 0);
    if (d.kind == OUT_GLU) {
        // fragments 2p (gate) and 2p+1 (up) hold the same output columns
        uint16_t *o = reinterpret_cast<uint16_t *>(d.ptr);
#pragma unroll
        for (int p = 0; p < TL_NF / 2; p++) {
            if (!nval[2 * p + 1])
                continue;
            const int oc = (n0 - d.col0) / 2 + p * 16 + 4 * q;
#pragma unroll
            for (int f = 0; f < NMF; f++) {
                const int r = rbase + f * 16;
                if (r >= m1)
                    continue;
                float hf[4];
#pragma unroll
                for (int i = 0; i < 4; i++)
                    hf[i] = silu_f32(acc[f][2 * p][i]) * acc[f][2 * p + 1][i];
                const uint2 hv = make_uint2(pack_bf16x2(hf[0], hf[1]), pack_bf16x2(hf[2], hf[3]));
                uint16_t *dst = o + (int64_t)r * d.ld + oc;
                if (vec) {
                    *reinterpret_cast<uint2 *>(dst) = hv;
                } else {
                    dst[0] = (uint16_t)hv.x;
                    dst[1] = (uint16_t)(hv.x >> 16);
                    dst[2] = (uint16_t)hv.y;
                    dst[3] = (uint16_t)(hv.y >> 16);
                }
            }
        }
    } else {
#pragma unroll
        for (int nf = 0; nf < TL_NF; nf++) {
            const int n = n0 + nf * 16 + 4 * q;                  // first of this lane's 4 columns
            if (!nval[nf] || n >= d.n_valid)
                continue;
            const bool full = vec && n + 3 < d.n_valid;
            float bias[4] = {0.f, 0.f, 0.f, 0.f};
            if (d.kind == OUT_F32 && d.bias)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    bias[i] = (n + i < d.n_valid) ? d.bias[n + i] : 0.f;
#pragma unroll
            for (int f = 0; f < NMF; f++) {
                const int r = rbase + f * 16;
                if (r >= m1)
                    continue;
                if (d.kind == OUT_F32) {
                    float *dst = reinterpret_cast<float *>(d.ptr) + (int64_t)r * d.ld + (n - d.col0);
                    if (full) {
                        *reinterpret_cast<f32x4_t *>(dst) = f32x4_t{acc[f][nf][0] + bias[0], acc[f][nf][1] + bias[1],
                                                                   acc[f][nf][2] + bias[2], acc[f][nf][3] + bias[3]};
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            if (n + i < d.n_valid)
                                dst[i] = acc[f][nf][i] + bias[i];
                    }
                } else {
                    uint16_t *dst = reinterpret_cast<uint16_t *>(d.ptr) + (int64_t)r * d.ld + (n - d.col0);
                    if (full) {
                        *reinterpret_cast<uint2 *>(dst) =
                            make_uint2(pack_bf16x2(acc[f][nf][0], acc[f][nf][1]),
                                       pack_bf16x2(acc[f][nf][2], acc[f][nf][3]));
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            if (n + i < d.n_valid)
                                dst[i] = (uint16_t)f32_to_bf16_bits(acc[f][nf][i]);
                    }
                }
            }
        }
    }
}

template <bool MX>
__global__ __launch_bounds__(WAVE * 4) __attribute__((amdgpu_waves_per_eu(2, 2))) void tiled_kernel(const GemmArgs g, int gx, int gy)
{
    __shared__ u32x4_t lds[2][TL_SLOTS];
    int bx, by;
    if (!tiled_item(g, gx, gy, bx, by))
        return;
    int group = 0, m0, m1;
    if (g.tiles) {
        const int4 t = reinterpret_cast<const int4 *>(g.tiles + TILE_HEADER_INTS)[by];
        group = t.x;
        m0 = t.y;
        m1 = t.z;
    } else {
        m0 = by * TL_BM;
        m1 = min(g.M, m0 + TL_BM);
    }
    // one code path per workgroup, chosen by the tile's row count
    const int nmf = __builtin_amdgcn_readfirstlane((m1 - m0 + 15) / 16);
    if (nmf <= 2)
        tiled_tile<MX, 2>(g, bx, group, m0, m1, lds);
    else if (nmf == 3)
        tiled_tile<MX, 3>(g, bx, group, m0, m1, lds);
    else if (nmf == 4)
        tiled_tile<MX, 4>(g, bx, group, m0, m1, lds);
    else if (nmf == 5)
        tiled_tile<MX, 5>(g, bx, group, m0, m1, lds);
    else if (nmf == 6)
        tiled_tile<MX, 6>(g, bx, group, m0, m1, lds);
    else
        tiled_tile<MX, 8>(g, bx, group, m0, m1, lds);
}

template <bool MX>
static hipError_t launch_tiled_t(const GemmArgs &g, int grid_m, hipStream_t st)
{
    const int gx = (g.N + TL_BN - 1) / TL_BN;
    const int64_t grid = ((int64_t)gx * grid_m + TL_XCDS - 1) / TL_XCDS * TL_XCDS;
    if (grid > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((tiled_kernel<MX>), dim3((unsigned)grid), dim3(WAVE * 4), 0, st, g, gx, grid_m);
    return hipGetLastError();
}

// ---- Ring product: dense BF16 C = A . B^T for many rows (M >= 256) with both operands staged
// through LDS. K advances in 32-input stages; RG_NBUF stages are resident in LDS, each holding the
// operand-order 1 KiB blocks of A (16 rows each) and of B (the packed fragment blocks). Both are
// moved by direct global->LDS loads -- one wave instruction fills one 1 KiB block, no register round
// trip -- issued RG_NBUF - 1 stages ahead; a wave waits for its own loads of the next stage (vmcnt)
// and a barrier makes every wave's loads visible. K must be a multiple of 32.
// Two tile shapes, both eight waves at two per SIMD:
//  * 256 x 256 (2 x 4 waves of 128 x 64): every product; N and the output region boundaries must
//    be multiples of 64 columns so that a wave's columns lie in one region;
//  * 256 x 224 (4 x 2 waves of 64 x 112): single-region, non-GLU outputs, chosen when it fills the
//    last round of workgroups better -- e.g. 8192 x 7168 outputs are 896 tiles of 256 x 256 (3.5
//    rounds of 256 CUs, the last one half idle) but 1024 tiles of 256 x 224 (four full rounds, each
//    tile 7/8 of the work).
constexpr int RG_BM = 256, RG_BN = 256;
constexpr int RG_NBUF = 4;
constexpr int RG_WAVES = 8;

// NWM x (8 / NWM) waves, each WMF x WNF fragments of 16 x 16 outputs (measured for the square tile:
// eight waves of 128 x 64 at 1.07 PFLOP/s against 0.82 for four waves of 128 x 128 at one wave per
// SIMD with the next stage's fragments read during the MFMAs).
template <int NWM, int WMF, int WNF>
__global__ __launch_bounds__(WAVE *RG_WAVES) void ring_kernel(const GemmArgs g, int gx, int gy)
{
    constexpr int NW = RG_WAVES, NWN = NW / NWM;
    constexpr int BM = NWM * WMF * 16, BN = NWN * WNF * 16;
    constexpr int AF = BM / 16, BF = BN / 16;            // A and B blocks per stage
    constexpr int LOADS = (AF + BF + NW - 1) / NW;       // loads per wave per stage
    constexpr int AW = AF / LOADS;                       // the first AW waves load A, the rest B
    static_assert(AF % LOADS == 0 && BF <= (NW - AW) * LOADS, "stage blocks must split over the waves");
    __shared__ u32x4_t lds[RG_NBUF][AF + BF][WAVE];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const int wm = wv / NWN, wn = wv % NWN;
    int bx, by;
    if (!tiled_item(g, gx, gy, bx, by))
        return;
    // The last tile of each axis is shifted back to end at M (N): it overlaps its neighbour and
    // recomputes identical values in the same order, so no load or store leaves the matrices.
    const int m0 = min(by * BM, g.M - BM), n0 = min(bx * BN, g.N - BN);
    const int nst = g.K / BF16_STEP;

    // This wave's loads: blocks wv*LOADS .. wv*LOADS+LOADS-1 of a stage. Within a stage they are one
    // base plus a fixed stride: 16 rows of A, or one row-block stride of B's current 16-step chunk.
    // An A block (16 rows x 64 bytes) is loaded with four consecutive lanes on one row -- lane l
    // takes row r = l / 4 and 16-byte chunk (l % 4) ^ chunk_swizzle(r), so slot 4 r + (c ^
    // chunk_swizzle(r)) holds chunk c of row r -- which L2 serves at ~1.6x the rate of the operand
    // order (lane l on row l % 16); the fragment reads (lane l: row l % 16, chunk l / 16) then fall in
    // distinct banks.
    // When the B blocks do not fill the last wave, its spare loads repeat the last block (the same
    // bytes into the same slot), so that every wave issues the same number of loads.
    const bool loads_a = wv < AW;
    const int li = loads_a ? wv : wv - AW;
    const int bfirst = li * LOADS;                       // first B block of a B wave
    const uint8_t *a_base = reinterpret_cast<const uint8_t *>(
        g.A + (int64_t)(m0 + li * (LOADS * 16) + (lane >> 2)) * g.lda + 8 * ((lane & 3) ^ chunk_swizzle(lane >> 2)));
    const int bnb0 = n0 / 16 + bfirst;
    auto issue = [&](int s) {                // stage min(s, nst - 1) into buffer s % RG_NBUF
        const int ss = min(s, nst - 1), buf = s % RG_NBUF;
        const uint8_t *base;
        int64_t stride;
        if (loads_a) {
            base = a_base + ss * (BF16_STEP * 2);
            stride = 16 * g.lda * 2;
        } else {
            const int64_t rest = nst - ss / BF16_CHUNK_STEPS * BF16_CHUNK_STEPS;
            base = g.B + bf16_block_index(bnb0, ss, g.N, g.K) * BF16_BLOCK_BYTES + lane * 16;
            stride = (rest < BF16_CHUNK_STEPS ? rest : BF16_CHUNK_STEPS) * BF16_BLOCK_BYTES;
        }
#pragma unroll
        for (int i = 0; i < LOADS; i++) {
            const int bi = loads_a ? i : min(i, BF - 1 - bfirst);
            __builtin_amdgcn_global_load_lds(base + bi * stride,
                                             (__attribute__((address_space(3))) void *)&lds[buf][wv * LOADS + bi][0],
                                             16, 0, 0);
        }
    };

    f32x4_t acc[WMF][WNF];
#pragma unroll
    for (int f = 0; f < WMF; f++)
#pragma unroll
        for (int j = 0; j < WNF; j++)
            acc[f][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto read_frags = [&](int s, u32x4_t *bf, u32x4_t *af) {
        const int buf = s % RG_NBUF;
#pragma unroll
        for (int j = 0; j < WNF; j++)
            bf[j] = lds[buf][AF + wn * WNF + j][lane];
        const int rr = lane & 15, cc = lane >> 4;
#pragma unroll
        for (int f = 0; f < WMF; f++)
            af[f] = lds[buf][wm * WMF + f][rr * 4 + (cc ^ chunk_swizzle(rr))];
    };
    // Wait until only the later stages' loads of this wave are outstanding, then a barrier makes every
    // wave's loads of this stage visible (and all waves are past the previous stage).
    auto sync_stages = [&]() {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((RG_NBUF - 2) * LOADS));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto mma = [&](const u32x4_t *bc, const u32x4_t *ac) {
#pragma unroll
        for (int j = 0; j < WNF; j++)
#pragma unroll
            for (int f = 0; f < WMF; f++)
                acc[f][j] = mfma16(as_bf16x8(bc[j]), as_bf16x8(ac[f]), acc[f][j]);
    };
#pragma unroll
    for (int s = 0; s < RG_NBUF - 1; s++)
        issue(s);
    // A wave issues its loads and fragment reads at a raised priority and its matrix-core
    // instructions at the normal one: a wave's loads and fragment reads then go ahead of the
    // multiplies of the other wave on its SIMD (output product 468 -> 449-456 us, router + x-side
    // unchanged; the same in the grouped gate|up kernel made it slower).
    for (int s = 0; s < nst; s++) {
        sync_stages();                        // stage s landed for every wave; buffer s - 1 free
        __builtin_amdgcn_s_setprio(1);
        issue(s + RG_NBUF - 1);
        u32x4_t bc[WNF], ac[WMF];
        read_frags(s, bc, ac);
        __builtin_amdgcn_s_setprio(0);
        mma(bc, ac);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no load may land in LDS after the workgroup ends

    // Epilogue: lane (q, c) of fragment (f, j) holds row 16 f + c and columns 16 j + 4 q .. +3.
    const int n0w = n0 + wn * (WNF * 16);
    if (n0w >= g.N)
        return;
    const OutDesc d = out_region(g, n0w);
    const int q = lane >> 4;
    const int rbase = m0 + wm * (WMF * 16) + (lane & 15);
    if (d.kind == OUT_GLU) {
        uint16_t *o = reinterpret_cast<uint16_t *>(d.ptr);
#pragma unroll
        for (int p = 0; p < WNF / 2; p++) {
            if (n0w + 32 * p + 32 > g.N)
                break;
            const int oc = (n0w - d.col0) / 2 + p * 16 + 4 * q;
#pragma unroll
            for (int f = 0; f < WMF; f++) {
                const int r = rbase + f * 16;
                float hf[4];
#pragma unroll
                for (int i = 0; i < 4; i++)
                    hf[i] = silu_f32(acc[f][2 * p][i]) * acc[f][2 * p + 1][i];
                *reinterpret_cast<uint2 *>(o + (int64_t)r * d.ld + oc) =
                    make_uint2(pack_bf16x2(hf[0], hf[1]), pack_bf16x2(hf[2], hf[3]));
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < WNF; j++) {
        const int n = n0w + j * 16 + 4 * q;
        if (n >= d.n_valid)
            continue;
        const bool full = n + 3 < d.n_valid;
        float bias[4] = {0.f, 0.f, 0.f, 0.f};
        if (d.kind == OUT_F32 && d.bias)
#pragma unroll
            for (int i = 0; i < 4; i++)
                bias[i] = (n + i < d.n_valid) ? d.bias[n + i] : 0.f;
#pragma unroll
        for (int f = 0; f < WMF; f++) {
            const int r = rbase + f * 16;
            if (d.kind == OUT_F32) {
                float *dst = reinterpret_cast<float *>(d.ptr) + (int64_t)r * d.ld + (n - d.col0);
                if (full) {
                    *reinterpret_cast<f32x4_t *>(dst) = f32x4_t{acc[f][j][0] + bias[0], acc[f][j][1] + bias[1],
                                                               acc[f][j][2] + bias[2], acc[f][j][3] + bias[3]};
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (n + i < d.n_valid)
                            dst[i] = acc[f][j][i] + bias[i];
                }
            } else {
                uint16_t *dst = reinterpret_cast<uint16_t *>(d.ptr) + (int64_t)r * d.ld + (n - d.col0);
                if (full) {
                    *reinterpret_cast<uint2 *>(dst) =
                        make_uint2(pack_bf16x2(acc[f][j][0], acc[f][j][1]),
                                   pack_bf16x2(acc[f][j][2], acc[f][j][3]));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (n + i < d.n_valid)
                            dst[i] = (uint16_t)f32_to_bf16_bits(acc[f][j][i]);
                }
            }
        }
    }
}

constexpr int RG_NARROW_BN = 224;

bool ring_supported(const GemmArgs &g)
{
    auto out_ok = [](const OutDesc &d) {
        return d.ld % 4 == 0 && d.col0 % 4 == 0 && reinterpret_cast<uintptr_t>(d.ptr) % 16 == 0;
    };
    // every wave's 64 columns (the shifted last tile included) lie in one output region
    const bool two = g.split < g.N, three = g.split2 > 0 && g.split2 < g.N;
    return !g.tiles && !g.a_index && g.M >= RG_BM && g.N >= RG_BN && g.K > 0 && g.K % BF16_STEP == 0 &&
           g.lda % 8 == 0 && reinterpret_cast<uintptr_t>(g.A) % 16 == 0 && out_ok(g.lo) &&
           (g.N % 64 == 0 || (!two && !three && g.N % 16 == 0)) && (!two || (g.split % 64 == 0 && out_ok(g.hi))) &&
           (!three || (two && g.split2 > g.split && g.split2 % 64 == 0 && out_ok(g.top)));
}

// Ring tiles fill the GPU (256 CUs) only from 256 tiles on; below that (e.g. the router's 896
// columns) the 128 x 256 tiled kernel keeps more CUs busy.
bool ring_preferred(const GemmArgs &g)
{
    return ring_supported(g) && (int64_t)((g.M + RG_BM - 1) / RG_BM) * ((g.N + RG_BN - 1) / RG_BN) >= 256;
}

// The narrow tile serves one output region that is not a GLU; it is taken when whole rounds of
// workgroups times the tile's work come out below the square tile's (ties keep the square tile).
static bool ring_narrow(const GemmArgs &g, int cus)
{
    const bool one_region = g.split >= g.N && !(g.split2 > 0 && g.split2 < g.N);
    if (!one_region || g.lo.kind == OUT_GLU || g.N < RG_NARROW_BN || cus < 1)
        return false;
    auto cost = [&](int bn) {
        const int64_t tiles = (int64_t)((g.M + RG_BM - 1) / RG_BM) * ((g.N + bn - 1) / bn);
        return (tiles + cus - 1) / cus * bn;
    };
    return cost(RG_NARROW_BN) < cost(RG_BN);
}

hipError_t launch_ring(const GemmArgs &g, hipStream_t st)
{
    if (!ring_supported(g))
        return hipErrorInvalidValue;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return e;
    const bool narrow = ring_narrow(g, cus);
    const int bn = narrow ? RG_NARROW_BN : RG_BN;
    const int gx = (g.N + bn - 1) / bn, gy = (g.M + RG_BM - 1) / RG_BM;
    const int64_t grid = ((int64_t)gx * gy + TL_XCDS - 1) / TL_XCDS * TL_XCDS;
    if (grid > INT32_MAX)
        return hipErrorInvalidValue;
    if (narrow)
        hipLaunchKernelGGL((ring_kernel<4, 4, 7>), dim3((unsigned)grid), dim3(WAVE * RG_WAVES), 0, st, g, gx, gy);
    else
        hipLaunchKernelGGL((ring_kernel<2, 8, 4>), dim3((unsigned)grid), dim3(WAVE * RG_WAVES), 0, st, g, gx, gy);
    return hipGetLastError();
}

// ---- A-stationary grouped MXFP4 product for short K (the down projection, K = I <= 512).
// The workgroup stages its whole 128-row A tile (gathered rows, 128 x K BF16, at most 128 KiB) into
// LDS once, in the operand order above, with direct global->LDS loads (one wave instruction fills
// one 1 KiB block), then walks its run of 256-column N blocks. Eight waves, two per SIMD so that one
// wave's output stores and B waits overlap the other's matrix-core work: wave (mh, wn) owns rows
// 64 mh .. 64 mh + 63 and columns 64 wn .. 64 wn + 63 of every N block (4 x 4 fragments, 64
// accumulators per lane). When every valid row lies in the first 64 (an expert's short last tile),
// the two row halves take alternate N blocks instead. Each wave's MXFP4 B is loaded one 128-input
// block ahead (across N blocks too) while the current one multiplies. (At one wave per SIMD -- four
// waves of 128 x 64 -- the kernel ran at half the rate; eight waves of 128 x 64 spill.)
// Work is mapped XCD-major: the eight XCDs each take a contiguous run of the (tile, N-run) items
// counted on the device, so the tiles of one expert share an L2.
constexpr int AS_WAVES = 8, AS_WN = 4, AS_BN = AS_WN * TL_WAVE_N, AS_MF = 8, AS_NF = 4, AS_XCDS = 8;
constexpr int AS_STAGE_PITCH = 144;                     // bytes per staged output row (128 + 16 padding)
constexpr int AS_STAGE_BYTES = 16 * AS_STAGE_PITCH;      // one 16-row fragment of one wave

// One (tile, N-run) item whose rows need only the first NMF 16-row fragments.
template <int KB, int NMF>
__device__ __attribute__((always_inline)) inline void astat_item(const GemmArgs &g, int group, int m0, int m1, int j0,
                                                                 int j1, u32x4_t *lds, uint8_t *stage_all)
{
    constexpr int KS = KB * TL_SUB;                              // 32-wide sub-steps
    constexpr int WF = NMF > 4 ? 4 : NMF;                        // row fragments per wave
    constexpr int JSTEP = NMF > 4 ? 1 : 2;                       // N blocks are split between row halves
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const int wn = wv % AS_WN, mh = wv / AS_WN;
    const int fb = NMF > 4 ? mh * 4 : 0;                         // this wave's first row fragment
    const int jb = NMF > 4 ? j0 : j0 + mh;                       // this wave's first N block
    uint8_t *stage = stage_all + wv * AS_STAGE_BYTES;

    // A tile -> LDS as whole 128-byte lines: row-half h of fragment f, line L (inputs 64 L .. 64 L +
    // 63) is one 1 KiB block at (f * KS / 2 + L) * 2 + h, 8 rows x 128 bytes, row r8's 16-byte chunk
    // c at position c ^ r8 (the operand reads, rows 0..7 of one chunk at a time, then fall in
    // distinct banks). Only the NMF fragments that hold valid rows are loaded.
    for (int b = wv; b < KS * NMF; b += AS_WAVES) {
        const int f = b % NMF, L = (b / NMF) / 2, h = (b / NMF) % 2;
        const int r8 = lane >> 3;
        const int r = min(m0 + f * 16 + h * 8 + r8, m1 - 1);      // clamped valid row, never stored
        const int64_t row = g.a_index ? (int64_t)(g.a_index[r] / g.a_div) : (int64_t)r;
        __builtin_amdgcn_global_load_lds(g.A + row * g.lda + L * 64 + 8 * ((lane & 7) ^ r8),
                                         (__attribute__((address_space(3))) void *)&lds[((f * (KS / 2) + L) * 2 + h) * WAVE],
                                         16, 0, 0);
    }

    const uint8_t *Bg = g.B + (int64_t)group * g.b_stride;
    const int nbmax = g.N / 16 - 1;
    // B is prefetched one 128-input block ahead (the next block of this N block, or the first of the
    // wave's next N block), so a wave holds two blocks of B at a time. These are cached loads: every
    // tile of an expert reads the expert's whole matrix, and a popular expert has dozens of tiles
    // (8192 tokens: 408 -> 391 us against non-temporal loads).
    auto load_kb = [&](int j, int kb, u32x4_t *codes, uint32_t *sc) {
#pragma unroll
        for (int nf = 0; nf < AS_NF; nf++) {
            const int nb = min((j * AS_BN + wn * TL_WAVE_N) / 16 + nf, nbmax);
            const uint8_t *p = Bg + ((int64_t)nb * KB + kb) * MX_BLOCK_BYTES;
            codes[nf] = load16(p + lane * 16);
            sc[nf] = *reinterpret_cast<const uint32_t *>(p + MX_CODE_BYTES + 4 * (lane & 15));
        }
    };
    u32x4_t bc[AS_NF];
    uint32_t bs[AS_NF];
    load_kb(min(jb, j1 - 1), 0, bc, bs);
    __builtin_amdgcn_s_waitcnt(0);                               // A tile (and first B) have landed
    __syncthreads();

    const OutDesc d = g.lo;
    const int q = lane >> 4;
    uint16_t *out = reinterpret_cast<uint16_t *>(d.ptr);
    for (int j = jb; j < j1; j += JSTEP) {
        f32x4_t acc[WF][AS_NF];
#pragma unroll
        for (int f = 0; f < WF; f++)
#pragma unroll
            for (int nf = 0; nf < AS_NF; nf++)
                acc[f][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; kb++) {
            u32x4_t bn[AS_NF];
            uint32_t bsn[AS_NF];
            if (kb + 1 < KB)
                load_kb(j, kb + 1, bn, bsn);
            else
                load_kb(min(j + JSTEP, j1 - 1), 0, bn, bsn);
#pragma unroll
            for (int s = 0; s < TL_SUB; s++) {
                u32x4_t a[WF];
                const int ss = kb * TL_SUB + s, ar = lane & 15;                 // sub-step, operand row
                const int ac = ((ss % 2) * 4 + (lane >> 4)) ^ (ar & 7);         // position of its chunk
#pragma unroll
                for (int f = 0; f < WF; f++)
                    a[f] = lds[(((fb + f) * (KS / 2) + ss / 2) * 2 + (ar >> 3)) * WAVE + (ar & 7) * 8 + ac];
#pragma unroll
                for (int nf = 0; nf < AS_NF; nf++) {
                    const bf16x8_t b = mx_dequant8(bc[nf][s], e8m0_to_f32((bs[nf] >> (8 * s)) & 0xFFu));
#pragma unroll
                    for (int f = 0; f < WF; f++)
                        acc[f][nf] = mfma16(b, as_bf16x8(a[f]), acc[f][nf]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int nf = 0; nf < AS_NF; nf++) {
                bc[nf] = bn[nf];
                bs[nf] = bsn[nf];
            }
        }
        // lane (q, c) of fragment (f, nf) holds row (fb + f)*16 + c, columns nf*16 + 4q .. +3. The
        // outputs leave through this wave's LDS staging area, one 16-row fragment at a time, so
        // that each store instruction writes eight whole 128-byte row segments (32-byte pieces at
        // the 7 KiB row stride stored at a quarter of the rate).
        // Rows past the tile end, and a column slice past N, fall outside the store window.
        const int n0w = j * AS_BN + wn * TL_WAVE_N;
        const int rbase = m0 + fb * 16;
        const int wrows = n0w < d.n_valid ? max(0, min(m1 - rbase, WF * 16)) : 0;
        const auto win = row_window(wrows > 0 ? out + (int64_t)rbase * d.ld + n0w : out, wrows, d.ld);
#pragma unroll
        for (int f = 0; f < WF; f++) {
#pragma unroll
            for (int nf = 0; nf < AS_NF; nf++)
                *reinterpret_cast<uint2 *>(stage + (lane & 15) * AS_STAGE_PITCH + nf * 32 + 8 * q) =
                    make_uint2(pack_bf16x2(acc[f][nf][0], acc[f][nf][1]),
                               pack_bf16x2(acc[f][nf][2], acc[f][nf][3]));
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int rr = h * 8 + (lane >> 3);
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(stage + rr * AS_STAGE_PITCH + (lane & 7) * 16);
                store16_window<CPOL_NT>(v, win, ((f * 16 + rr) * d.ld + (lane & 7) * 8) * 2);
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

template <int KB>
__global__ __launch_bounds__(WAVE * AS_WAVES) void astat_kernel(const GemmArgs g, int nsplit)
{
    __shared__ u32x4_t lds[KB * TL_SUB * AS_MF * WAVE];
    __shared__ __attribute__((aligned(16))) uint8_t stage[AS_WAVES * AS_STAGE_BYTES];
    const int total = g.tiles[0] * nsplit;
    const int per = (total + AS_XCDS - 1) / AS_XCDS;
    const int slot = blockIdx.x / AS_XCDS;
    const int item = (blockIdx.x % AS_XCDS) * per + slot;
    if (slot >= per || item >= total)
        return;
    const int4 t = reinterpret_cast<const int4 *>(g.tiles + TILE_HEADER_INTS)[item / nsplit];
    const int part = item % nsplit;
    const int nbn = (g.N + AS_BN - 1) / AS_BN;
    const int j0 = part * nbn / nsplit, j1 = (part + 1) * nbn / nsplit;
    if (j0 >= j1)
        return;
    // one code path per workgroup, chosen by the tile's row count
    const int nmf = __builtin_amdgcn_readfirstlane((t.z - t.y + 15) / 16);
    if (nmf <= 2)
        astat_item<KB, 2>(g, t.x, t.y, t.z, j0, j1, lds, stage);
    else if (nmf <= 4)
        astat_item<KB, 4>(g, t.x, t.y, t.z, j0, j1, lds, stage);
    else
        astat_item<KB, 8>(g, t.x, t.y, t.z, j0, j1, lds, stage);
}

template <int KB>
static hipError_t launch_astat_t(const GemmArgs &g, int max_tiles, hipStream_t st)
{
    const int nbn = (g.N + AS_BN - 1) / AS_BN;
    // enough (tile, N-run) items for ~8 rounds of 256 workgroups at the largest tile count
    const int nsplit = std::max(1, std::min(nbn, (2048 + max_tiles - 1) / max_tiles));
    const int64_t items = (int64_t)max_tiles * nsplit;
    const int64_t grid = (items + AS_XCDS - 1) / AS_XCDS * AS_XCDS;
    if (grid > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((astat_kernel<KB>), dim3((unsigned)grid), dim3(WAVE * AS_WAVES), 0, st, g, nsplit);
    return hipGetLastError();
}

bool astat_supported(const GemmArgs &g)
{
    const OutDesc &d = g.lo;
    // whole 64-column wave slices are stored with 16-byte writes
    return g.tiles && g.K % MX_STEP == 0 && g.K >= MX_STEP && g.K <= AS_MAX_K && g.N % 64 == 0 && g.N > 0 &&
           g.split >= g.N && d.kind == OUT_BF16 && d.col0 == 0 && d.n_valid == g.N && d.ld % 8 == 0 &&
           d.ld >= g.N && reinterpret_cast<uintptr_t>(d.ptr) % 16 == 0 && g.lda % 8 == 0 &&
           reinterpret_cast<uintptr_t>(g.A) % 16 == 0;
}

hipError_t launch_astat(const GemmArgs &g, int max_tiles, hipStream_t st)
{
    if (!astat_supported(g))
        return hipErrorInvalidValue;
    if (max_tiles <= 0)
        return hipSuccess;
    switch (g.K / MX_STEP) {
    case 1: return launch_astat_t<1>(g, max_tiles, st);
    case 2: return launch_astat_t<2>(g, max_tiles, st);
    case 3: return launch_astat_t<3>(g, max_tiles, st);
    case 4: return launch_astat_t<4>(g, max_tiles, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_tiled(const GemmArgs &g, bool mx, int max_tiles, hipStream_t st)
{
    if (g.N % 16 || g.N <= 0 || g.K % (mx ? MX_STEP : BF16_STEP) || g.K <= 0)
        return hipErrorInvalidValue;
    if ((g.split < g.N && g.split % 64) || (g.split2 > 0 && (g.split2 % 64 || g.split2 <= g.split)))
        return hipErrorInvalidValue;   // a wave's 64 columns must lie in one output region
    const int grid_m = g.tiles ? max_tiles : (g.M + TILED_BM - 1) / TILED_BM;
    if (grid_m <= 0)
        return hipSuccess;
    return mx ? launch_tiled_t<true>(g, grid_m, st) : launch_tiled_t<false>(g, grid_m, st);
}

} // namespace mxmoe
