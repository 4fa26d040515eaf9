// combine.hip -- the tile list of the grouped expert GEMMs and the fixed-order gate-weighted
// combine of the expert outputs.
#include "kernels.hpp"

namespace mxmoe {

__global__ __launch_bounds__(1024) void tilemap_kernel(const int32_t *__restrict__ offsets, int E, int bm,
                                                       int32_t *__restrict__ tiles)
{
    __shared__ int sh[16];
    write_tiles(offsets, E, bm, tiles, sh);
}

hipError_t launch_tilemap(const int32_t *offsets, int E, int bm, int32_t *tiles, hipStream_t st)
{
    hipLaunchKernelGGL(tilemap_kernel, dim3(1), dim3(1024), 0, st, offsets, E, bm, tiles);
    return hipGetLastError();
}

// zc[t, c] = bf16(sum over slots j = 0..K-1, in order, of w[t, j] * Y[inv[t K + j], c]).
// Each thread owns 8 consecutive columns of one token (16-byte loads and store); FP32 sums. Slots
// go in batches of CB: the batch's rows and weights, then all its row loads, are issued before any
// is used, so a wave keeps CB loads in flight; the sums still run in slot order. The rows of y are
// read once, with non-temporal loads (at 8192 tokens, 940 MB: 236 -> 178 us against cached loads).
constexpr int CB = 8;
__global__ __launch_bounds__(64) void combine_kernel(const uint16_t *__restrict__ Y, int Lt,
                                                     const int32_t *__restrict__ inv, const float *__restrict__ w,
                                                     int K, uint16_t *__restrict__ out, int64_t ldo, int chunks)
{
    const int t = (int)(blockIdx.x / chunks);
    const int c8 = (int)(blockIdx.x % chunks) * 64 + threadIdx.x;
    if (c8 * 8 >= Lt)
        return;
    const int32_t *it = inv + (int64_t)t * K;
    const float *wt = w + (int64_t)t * K;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto add = [&](float wj, const u32x4_t &y) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            acc[2 * i] += wj * bf16_bits_to_f32(y[i] & 0xFFFFu);
            acc[2 * i + 1] += wj * bf16_bits_to_f32(y[i] >> 16);
        }
    };
    int j0 = 0;
    for (; j0 + CB <= K; j0 += CB) {
        int64_t r[CB];
        float wj[CB];
#pragma unroll
        for (int u = 0; u < CB; u++) {
            r[u] = it[j0 + u];
            wj[u] = wt[j0 + u];
        }
        u32x4_t y[CB];
#pragma unroll
        for (int u = 0; u < CB; u++)
            y[u] = load16_nt(Y + r[u] * Lt + c8 * 8);
#pragma unroll
        for (int u = 0; u < CB; u++)
            add(wj[u], y[u]);
    }
    for (; j0 < K; j0++)
        add(wt[j0], load16_nt(Y + (int64_t)it[j0] * Lt + c8 * 8));
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; i++)
        o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *reinterpret_cast<u32x4_t *>(out + (int64_t)t * ldo + c8 * 8) = o;
}

hipError_t launch_combine(const uint16_t *Y, int Lt, const int32_t *inv, const float *w, int T, int K,
                          uint16_t *out, int64_t ldo, hipStream_t st)
{
    // column chunks fastest: the chunks of one token (its K rows of y read whole) run back to back
    const int64_t chunks = (Lt / 8 + 63) / 64;
    if (T <= 0)
        return hipSuccess;
    if (chunks * T > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(chunks * T)), dim3(64), 0, st, Y, Lt, inv, w, K, out, ldo,
                       (int)chunks);
    return hipGetLastError();
}

} // namespace mxmoe
