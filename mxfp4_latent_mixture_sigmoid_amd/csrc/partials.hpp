// partials.hpp -- sums of split-K FP32 partial tiles (the few-token dense products' layout, see
// skinny_partial_index) and the x-side epilogue on them; shared by the epilogue kernels and the
// combined top-K / x-side epilogue launch.
#pragma once

#include "kernels.hpp"

namespace mxmoe {

// Partial sums load SUM_BATCH splits at a time (addresses clamped, so every load is valid) before
// any of them is used: one round of loads for up to 16 splits (K up to 8192 in 512-wide splits).
constexpr int SUM_BATCH = 16;
// Sum over the splits of one lane's 16-byte partial slot (four rows of one column), split order.
__device__ inline f32x4_t sum_slot(const float *slot, int64_t split_stride, int splits)
{
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < splits; s0 += SUM_BATCH) {
        f32x4_t t[SUM_BATCH];
#pragma unroll
        for (int u = 0; u < SUM_BATCH; u++)
            t[u] = *reinterpret_cast<const f32x4_t *>(slot + min(s0 + u, splits - 1) * split_stride);
#pragma unroll
        for (int u = 0; u < SUM_BATCH; u++)
            if (s0 + u < splits)
                v += t[u];
    }
    return v;
}

// x-side epilogue. Thread (nb, mf, lane) owns rows mf*16 + 4(lane/16) .. +3 of column
// nb*16 + lane%16: z = bf16(sum) for the latent blocks; for a shared-expert pair of blocks (16
// gate columns, then the matching 16 up columns) the thread of the gate block forms
// h_s = bf16(silu(gate) * up).
__device__ inline void xside_epi_item(const XsideEpiArgs &e, int64_t gid)
{
    const int lane = (int)(gid % WAVE);
    const int64_t frag = gid / WAVE;
    const int mf = (int)(frag % 4);
    const int nbz = e.Lt / 16, npairs = e.shared_cols / 32;
    const int64_t unit = frag / 4;                           // latent block, then shared pair
    if (unit >= nbz + npairs || mf * 16 >= e.M)
        return;
    const int col16 = lane & 15, r0 = mf * 16 + 4 * (lane >> 4);
    if (unit < nbz) {
        const f32x4_t v = sum_slot(e.P + (unit * 4 + mf) * (int64_t)SKINNY_TILE_FLOATS / 4 + lane * 4,
                                   e.p_split_stride, e.splits);
#pragma unroll
        for (int i = 0; i < 4; i++)
            if (r0 + i < e.M)
                e.z[(int64_t)(r0 + i) * e.Lt + unit * 16 + col16] = (uint16_t)f32_to_bf16_bits(v[i]);
    } else {
        const int pr = (int)(unit - nbz);
        const int64_t gb = nbz + 2 * pr;                     // gate block; up block is gb + 1
        const f32x4_t gv = sum_slot(e.P + (gb * 4 + mf) * (int64_t)SKINNY_TILE_FLOATS / 4 + lane * 4,
                                    e.p_split_stride, e.splits);
        const f32x4_t uv = sum_slot(e.P + ((gb + 1) * 4 + mf) * (int64_t)SKINNY_TILE_FLOATS / 4 + lane * 4,
                                    e.p_split_stride, e.splits);
#pragma unroll
        for (int i = 0; i < 4; i++)
            if (r0 + i < e.M)
                e.acat[(int64_t)(r0 + i) * e.ldcat + e.Lt + pr * 16 + col16] =
                    (uint16_t)f32_to_bf16_bits(silu_f32(gv[i]) * uv[i]);
    }
}

} // namespace mxmoe
