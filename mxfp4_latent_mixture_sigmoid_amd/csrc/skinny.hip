// skinny.hip -- dense BF16 products for a few tokens (T <= 64), where the weights must be streamed
// from HBM exactly once at full bandwidth.
//
// The product C[T, N] = A[T, K] . B[N, K]^T is cut into (column group, K chunk) work items, enough
// of them to occupy every CU. A workgroup first issues all of its weight loads (one 1 KiB fragment
// block per wave and 32-wide K step, straight into registers), then stages its activation chunk
// (T rows x chunk) in LDS once for all of its waves, and finally runs the 16x16x32 BF16 matrix-core
// instructions. Each item writes an FP32 partial tile; the kernel that consumes the product sums the
// partials of the K chunks in chunk order (fixed order: the result does not depend on scheduling)
// and applies the epilogue: router logits (+bias) in the top-K kernel, z and the shared-expert GLU
// in xside_epilogue_kernel, the final BF16 output in out_epilogue_kernel.
#include "kernels.hpp"
#include "partials.hpp"

#include <algorithm>

namespace mxmoe {


// LDS holds the activation chunk per step s and 16-row fragment mf in a 1 KiB block: slot
// 4 r + (c ^ chunk_swizzle(r)) holds 16-byte chunk c (inputs s*32 + 8c .. +7) of row mf*16 + r. The staging
// thread t of each 64 loads the chunk of slot t (four consecutive threads on one row, which L2
// serves faster than one thread per row) and writes slot t (sequential); the operand read of lane l
// (row l % 16, chunk l / 16) then falls in distinct banks.
template <int WAVES, int SK_MAX_STEPS>
__global__ __launch_bounds__(WAVE *WAVES) void skinny_kernel(const SkinnyArgs g)
{
    extern __shared__ u32x4_t lds_a[];   // [nsteps][4 fragments][64 lanes]
    const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
    if (g.zero_word && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
        *g.zero_word = 0u;
    const int split = blockIdx.y;
    const int kc0 = split * SK_MAX_STEPS * BF16_STEP;
    const int nsteps = min(SK_MAX_STEPS * BF16_STEP, g.K - kc0) / BF16_STEP;
    const int mt = (g.M + 15) / 16;
    const int nb = blockIdx.x * WAVES + wv;           // this wave's 16-row block of B
    const bool active = nb < g.N / 16;

    // 1. Weight stream: every fragment of this wave's chunk, issued before anything waits (idle
    //    waves re-read the last valid block; their result is never used). The empty asm with a
    //    memory clobber keeps the compiler from sinking these loads below the LDS staging.
    u32x4_t b[SK_MAX_STEPS];
    {
        const int nbc = min(nb, g.N / 16 - 1);
        const uint8_t *bp = g.B + bf16_block_index(nbc, kc0 / BF16_STEP, g.N, g.K) * BF16_BLOCK_BYTES + lane * 16;
#pragma unroll
        for (int s = 0; s < SK_MAX_STEPS; s++)
            b[s] = load16_nt(bp + min(s, nsteps - 1) * BF16_BLOCK_BYTES);
    }
    asm volatile("" ::: "memory");

    // 2. Activation chunk -> registers (all loads in flight together) -> LDS in operand order,
    //    rows >= M zero, shared by all waves of the workgroup.
    constexpr int A_PER_THREAD = SK_MAX_STEPS * 4 * WAVE / (WAVE * WAVES);
    u32x4_t av[A_PER_THREAD];
#pragma unroll
    for (int u = 0; u < A_PER_THREAD; u++) {
        const int slot = threadIdx.x + u * WAVE * WAVES;        // block (slot / 64), lane slot % 64
        const int blk = slot / WAVE, sl = slot % WAVE;
        const int st = min(blk / 4, nsteps - 1), m = (blk % 4) * 16 + (sl >> 2);
        av[u] = load16(g.A + (int64_t)min(m, g.M - 1) * g.lda + kc0 + st * BF16_STEP + 8 * ((sl & 3) ^ chunk_swizzle(sl >> 2)));
    }
#pragma unroll
    for (int u = 0; u < A_PER_THREAD; u++) {
        const int slot = threadIdx.x + u * WAVE * WAVES;
        const int blk = slot / WAVE, sl = slot % WAVE;
        const int m = (blk % 4) * 16 + (sl >> 2);
        if (blk / 4 < nsteps && (blk % 4) < mt)
            lds_a[slot] = m < g.M ? av[u] : u32x4_t{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    if (!active)
        return;

    // 3. Matrix-core products over the chunk: per step, all A fragments from LDS, then the MFMAs.
    f32x4_t acc[4];
#pragma unroll
    for (int mf = 0; mf < 4; mf++)
        acc[mf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SK_MAX_STEPS; s++) {
        if (s < nsteps) {
            u32x4_t a[4];
#pragma unroll
            for (int mf = 0; mf < 4; mf++)
                a[mf] = lds_a[(s * 4 + mf) * WAVE + (lane & 15) * 4 + ((lane >> 4) ^ chunk_swizzle(lane & 15))];
#pragma unroll
            for (int mf = 0; mf < 4; mf++)
                if (mf < mt)
                    acc[mf] = mfma16(as_bf16x8(a[mf]), as_bf16x8(b[s]), acc[mf]);
        }
    }

    // 4. FP32 partial tile of this K chunk in accumulator order (see skinny_partial_index): each
    //    lane stores its four values of a fragment as one 16-byte store, a wave 1 KiB contiguous.
    float *P = g.P + (int64_t)split * g.p_split_stride + (int64_t)nb * SKINNY_TILE_FLOATS;
#pragma unroll
    for (int mf = 0; mf < 4; mf++)
        if (mf < mt)
            *reinterpret_cast<f32x4_t *>(P + (mf * WAVE + lane) * 4) = acc[mf];
}

// Persistent variant: workgroup w owns K split (w % splits) -- a chunk of UNITS x 16 steps -- and the
// 16-row weight blocks nb = (w / splits) * WAVES + wave + j * (groups * WAVES), j = 0, 1, ... where
// groups = gridDim.x / splits. The activation chunk of its split is staged in LDS once; each wave
// then streams its blocks as 16-step units (one contiguous 16 KiB range each), loading the next unit
// while the current one is multiplied, and writes a block's partial tile after its last unit.
template <int WAVES, int UNITS, int MT>
__global__ __launch_bounds__(WAVE *WAVES) void skinny_persist_kernel(const SkinnyArgs g, int splits)
{
    constexpr int STEPS = 16, CSTEPS = STEPS * UNITS;
    __shared__ u32x4_t lds_a[CSTEPS * 4 * WAVE];   // [steps][4 fragments][64 lanes]
    const int lane = threadIdx.x & (WAVE - 1);
    if (g.zero_word && blockIdx.x == 0 && threadIdx.x == 0)
        *g.zero_word = 0u;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const int split = blockIdx.x % splits, grp = blockIdx.x / splits;
    const int groups = gridDim.x / splits;
    const int kc0 = split * CSTEPS * BF16_STEP;
    const int nsteps = min(CSTEPS * BF16_STEP, g.K - kc0) / BF16_STEP;
    const int nunits = (nsteps + STEPS - 1) / STEPS;
    const int nblocks = g.N / 16;
    const int stride = groups * WAVES;
    const int nb0 = grp * WAVES + wv;
    const int items = (nb0 < nblocks ? (nblocks - 1 - nb0) / stride + 1 : 0) * nunits;   // (block, unit)

    auto load_b = [&](int i, u32x4_t *b) {
        const int blk = min(nb0 + (i / nunits) * stride, nblocks - 1), s0 = (i % nunits) * STEPS;
        const uint8_t *bp =
            g.B + bf16_block_index(blk, kc0 / BF16_STEP + s0, g.N, g.K) * BF16_BLOCK_BYTES + lane * 16;
#pragma unroll
        for (int s = 0; s < STEPS; s++)
            b[s] = load16_nt(bp + min(s, nsteps - s0 - 1) * BF16_BLOCK_BYTES);
    };
    u32x4_t b0[STEPS], b1[STEPS];
    if (items > 0)
        load_b(0, b0);
    asm volatile("" ::: "memory");

    constexpr int A_PER_THREAD = CSTEPS * 4 * WAVE / (WAVE * WAVES);
    {
        u32x4_t av[A_PER_THREAD];
#pragma unroll
        for (int u = 0; u < A_PER_THREAD; u++) {
            const int slot = threadIdx.x + u * WAVE * WAVES;
            const int blk = slot / WAVE, sl = slot % WAVE;
            const int st = min(blk / 4, nsteps - 1), m = (blk % 4) * 16 + (sl >> 2);
            av[u] = load16(g.A + (int64_t)min(m, g.M - 1) * g.lda + kc0 + st * BF16_STEP + 8 * ((sl & 3) ^ chunk_swizzle(sl >> 2)));
        }
#pragma unroll
        for (int u = 0; u < A_PER_THREAD; u++) {
            const int slot = threadIdx.x + u * WAVE * WAVES;
            const int blk = slot / WAVE, sl = slot % WAVE;
            const int m = (blk % 4) * 16 + (sl >> 2);
            if (blk / 4 < nsteps && (blk % 4) < MT)
                lds_a[slot] = m < g.M ? av[u] : u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    __syncthreads();

    f32x4_t acc[4];
    auto compute = [&](int i, const u32x4_t *b) {
        const int unit = i % nunits;
        if (unit == 0)
#pragma unroll
            for (int mf = 0; mf < 4; mf++)
                acc[mf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < STEPS; s++) {
            const int step = unit * STEPS + s;
            if (step < nsteps) {
                u32x4_t a[4];
#pragma unroll
                for (int mf = 0; mf < 4; mf++)
                    a[mf] = lds_a[(step * 4 + mf) * WAVE + (lane & 15) * 4 + ((lane >> 4) ^ chunk_swizzle(lane & 15))];
#pragma unroll
                for (int mf = 0; mf < 4; mf++)
                    if (mf < MT)
                        acc[mf] = mfma16(as_bf16x8(a[mf]), as_bf16x8(b[s]), acc[mf]);
            }
        }
        if (unit == nunits - 1) {
            const int blk = nb0 + (i / nunits) * stride;
            float *P = g.P + (int64_t)split * g.p_split_stride + (int64_t)blk * SKINNY_TILE_FLOATS;
#pragma unroll
            for (int mf = 0; mf < 4; mf++)
                if (mf < MT)
                    *reinterpret_cast<f32x4_t *>(P + (mf * WAVE + lane) * 4) = acc[mf];
        }
    };

    // Two units per iteration, ping-ponging the register buffers.
    for (int i = 0; i < items; i += 2) {
        if (i + 1 < items)
            load_b(i + 1, b1);
        compute(i, b0);
        if (i + 1 >= items)
            break;
        if (i + 2 < items)
            load_b(i + 2, b0);
        compute(i + 1, b1);
    }
}

// chunk_steps is the K range of a split in 32-wide steps (16: one packed K chunk).
hipError_t launch_skinny_persist(const SkinnyArgs &g, int waves, int groups, int chunk_steps, hipStream_t st)
{
    if (g.M < 1 || g.M > SKINNY_MAX_M || g.N % 16 || g.K % BF16_STEP || groups < 1)
        return hipErrorInvalidValue;
    const int splits = skinny_splits(g.K, chunk_steps);
    const dim3 grid(splits * groups);
    const int mt = (g.M + 15) / 16;
#define MOE_PERSIST(W, U, MT)                                                                                        \
    if (waves == W && chunk_steps == 16 * U && mt == MT) {                                                          \
        hipLaunchKernelGGL((skinny_persist_kernel<W, U, MT>), grid, dim3(WAVE * W), 0, st, g, splits);               \
        return hipGetLastError();                                                                                    \
    }
    MOE_PERSIST(8, 1, 1)
    MOE_PERSIST(8, 1, 2)
    MOE_PERSIST(8, 1, 3)
    MOE_PERSIST(8, 1, 4)
#undef MOE_PERSIST
    return hipErrorInvalidValue;
}

int skinny_splits(int K, int chunk_steps)
{
    const int chunk = chunk_steps * BF16_STEP;
    return (K + chunk - 1) / chunk;
}

// One workgroup per (K split, group of `waves` 16-row blocks); chunk_steps (16: one packed K chunk)
// sets the K range of a split. Only (4 waves, 16 steps) is built: the router product alone.
hipError_t launch_skinny(const SkinnyArgs &g, int waves, int chunk_steps, hipStream_t st)
{
    if (g.M < 1 || g.M > SKINNY_MAX_M || g.N % 16 || g.K % BF16_STEP)
        return hipErrorInvalidValue;
    const int steps = std::min(chunk_steps * BF16_STEP, g.K) / BF16_STEP;
    const size_t lds = (size_t)steps * 4 * WAVE * 16;
    const dim3 grid((g.N / 16 + waves - 1) / waves, skinny_splits(g.K, chunk_steps));
#define MOE_SKINNY(W, S)                                                                                              \
    if (waves == W && chunk_steps == S) {                                                                             \
        hipLaunchKernelGGL((skinny_kernel<W, S>), grid, dim3(WAVE * W), lds, st, g);                                   \
        return hipGetLastError();                                                                                     \
    }
    MOE_SKINNY(4, 16)
#undef MOE_SKINNY
    return hipErrorInvalidValue;
}

// x-side epilogue over the whole partials (per-item work: xside_epi_item). With tile lists
// requested, one extra (last) workgroup builds them.
__global__ __launch_bounds__(256) void xside_epilogue_kernel(const XsideEpiArgs e)
{
    if (e.tiles && blockIdx.x == gridDim.x - 1) {
        __shared__ int sh[16];
        write_tiles(e.offsets, e.E, e.bm, e.tiles, sh);
        return;
    }
    xside_epi_item(e, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

hipError_t launch_xside_epilogue(const XsideEpiArgs &e, hipStream_t st)
{
    const int64_t threads = (int64_t)(e.Lt / 16 + e.shared_cols / 32) * 4 * WAVE;
    const unsigned blocks = (e.tiles ? 1 : 0) + (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(xside_epilogue_kernel, dim3(blocks), dim3(256), 0, st, e);
    return hipGetLastError();
}

// out = bf16(sum of partials). Thread (row quad q, column c) of a 64 x 16 tile reads the four
// values of rows 4q..4q+3 as one 16-byte load per split and writes the four BF16 results.
__global__ __launch_bounds__(256) void out_epilogue_kernel(const float *__restrict__ P, int64_t split_stride,
                                                           int splits, int M, int N, uint16_t *__restrict__ out)
{
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (nb, mf, lane)
    const int lane = (int)(gid % WAVE);
    const int64_t frag = gid / WAVE;
    const int mf = (int)(frag % 4);
    const int64_t nb = frag / 4;
    if (nb >= N / 16 || mf * 16 >= M)
        return;
    const float *src = P + gid * 4;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < splits; s0 += SUM_BATCH) {
        f32x4_t t[SUM_BATCH];
#pragma unroll
        for (int u = 0; u < SUM_BATCH; u++)
            t[u] = *reinterpret_cast<const f32x4_t *>(src + min(s0 + u, splits - 1) * split_stride);
#pragma unroll
        for (int u = 0; u < SUM_BATCH; u++)
            if (s0 + u < splits)
                v += t[u];
    }
    const int col = (int)nb * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int row = mf * 16 + 4 * (lane >> 4) + i;
        if (row < M)
            out[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_bits(v[i]);
    }
}

hipError_t launch_out_epilogue(const float *P, int64_t split_stride, int splits, int M, int N, uint16_t *out,
                               hipStream_t st)
{
    if (N % 16 || M < 1 || M > SKINNY_MAX_M)
        return hipErrorInvalidValue;
    const int64_t threads = (int64_t)(N / 16) * 4 * WAVE;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(out_epilogue_kernel, dim3(blocks), dim3(256), 0, st, P, split_stride, splits, M, N, out);
    return hipGetLastError();
}

} // namespace mxmoe
