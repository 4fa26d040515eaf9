// route.hip -- deterministic top-K selection with sigmoid gate weights, and the grouping of
// token/expert pairs by expert (histogram, per-expert scan, stable scatter).
#include "kernels.hpp"

#include <climits>

namespace mxmoe {

__device__ inline int wave_incl_scan(int v)
{
    const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const int t = __shfl_up(v, o);
        if (lane >= o)
            v += t;
    }
    return v;
}

// Exclusive prefix sum of one value per thread over the whole workgroup (blockDim <= 1024).
// `sh` holds >= 16 ints of LDS. Returns the prefix; *total receives the workgroup sum.
__device__ int block_excl_scan(int v, int *sh, int *total)
{
    const int lane = threadIdx.x & (WAVE - 1), wid = threadIdx.x / WAVE;
    const int nw = (blockDim.x + WAVE - 1) / WAVE;
    const int inc = wave_incl_scan(v);
    if (lane == WAVE - 1)
        sh[wid] = inc;
    __syncthreads();
    if (wid == 0) {
        int x = lane < nw ? sh[lane] : 0;
        x = wave_incl_scan(x);
        if (lane < nw)
            sh[lane] = x;
    }
    __syncthreads();
    const int base = wid ? sh[wid - 1] : 0;
    *total = sh[nw - 1];
    __syncthreads();
    return base + inc - v;
}

// Order used by the selection: larger logit first, equal logits by lower expert index.
__device__ inline bool before(float va, int ia, float vb, int ib) { return va > vb || (va == vb && ia < ib); }

// One wave per token. Each lane keeps the logits of experts lane, lane + 64, ...; K rounds of a
// wave-wide arg-max pick the experts in rank order. Gate weights: sigmoid of the selected
// logits, divided by their sum (a butterfly sum, bitwise identical in every lane).
template <int SLOTS>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E, int K,
                                                   int32_t *__restrict__ ids, float *__restrict__ w)
{
    const int lane = threadIdx.x & (WAVE - 1);
    const int t = blockIdx.x * 4 + threadIdx.x / WAVE;
    if (t >= T)
        return;
    const float *l = logits + (int64_t)t * E;
    float v[SLOTS];
    int idx[SLOTS];
#pragma unroll
    for (int j = 0; j < SLOTS; j++) {
        const int e = lane + WAVE * j;
        v[j] = e < E ? l[e] : -INFINITY;
        idx[j] = e < E ? e : INT_MAX;
    }
    int my_id = 0;
    float my_v = 0.f;
    for (int k = 0; k < K; k++) {
        float bv = v[0];
        int bi = idx[0];
#pragma unroll
        for (int j = 1; j < SLOTS; j++)
            if (before(v[j], idx[j], bv, bi)) {
                bv = v[j];
                bi = idx[j];
            }
#pragma unroll
        for (int o = WAVE / 2; o >= 1; o >>= 1) {
            const float ov = __shfl_xor(bv, o);
            const int oi = __shfl_xor(bi, o);
            if (before(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if (lane == k) {
            my_id = bi;
            my_v = bv;
        }
        if ((bi & (WAVE - 1)) == lane) {
#pragma unroll
            for (int j = 0; j < SLOTS; j++)
                if (j == (bi / WAVE)) {
                    v[j] = -INFINITY;
                    idx[j] = INT_MAX;
                }
        }
    }
    const float s = lane < K ? 1.0f / (1.0f + expf(-my_v)) : 0.0f;
    float sum = s;
#pragma unroll
    for (int o = WAVE / 2; o >= 1; o >>= 1)
        sum += __shfl_xor(sum, o);
    if (lane < K) {
        ids[(int64_t)t * K + lane] = my_id;
        w[(int64_t)t * K + lane] = s / sum;
    }
}

hipError_t launch_topk(const float *logits, int T, int E, int K, int32_t *ids, float *w, hipStream_t st)
{
    const dim3 grid((T + 3) / 4);
    if (E <= 2 * WAVE)
        hipLaunchKernelGGL(topk_kernel<2>, grid, dim3(256), 0, st, logits, T, E, K, ids, w);
    else if (E <= 16 * WAVE)
        hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, st, logits, T, E, K, ids, w);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// Pass 1: per block of tokens, the number of pairs routed to each expert -> hist[e * nb + b].
__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t *__restrict__ ids, int T, int K, int E,
                                                        int nb, int32_t *__restrict__ hist)
{
    extern __shared__ int cnt[];
    const int b = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        cnt[e] = 0;
    __syncthreads();
    const int p0 = b * PERM_TOKENS_PER_BLOCK * K;
    const int p1 = min(T, (b + 1) * PERM_TOKENS_PER_BLOCK) * K;
    for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x)
        atomicAdd(&cnt[ids[p]], 1);   // integer counts: independent of the order of the adds
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        hist[(int64_t)e * nb + b] = cnt[e];
}

// Pass 2: for each expert, exclusive scan of its per-block counts (in place) and its total.
__global__ __launch_bounds__(256) void perm_colscan_kernel(int32_t *__restrict__ hist, int nb,
                                                           int32_t *__restrict__ counts)
{
    __shared__ int sh[16];
    const int e = blockIdx.x;
    int32_t *row = hist + (int64_t)e * nb;
    const int per = (nb + blockDim.x - 1) / blockDim.x;
    const int i0 = threadIdx.x * per, i1 = min(nb, i0 + per);
    int local = 0;
    for (int i = i0; i < i1; i++)
        local += row[i];
    int total;
    int run = block_excl_scan(local, sh, &total);
    for (int i = i0; i < i1; i++) {
        const int c = row[i];
        row[i] = run;
        run += c;
    }
    if (threadIdx.x == 0)
        counts[e] = total;
}

// Pass 3: expert offsets (exclusive scan of counts), then a stable scatter: one wave walks the
// block's tokens in order; the K experts of a token are distinct, so its K lanes bump distinct
// LDS counters and every pair lands at offsets[e] + (pairs of e in earlier tokens).
__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t *__restrict__ ids, int T, int K, int E,
                                                           int nb, const int32_t *__restrict__ hist,
                                                           const int32_t *__restrict__ counts,
                                                           int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ sorted_pairs,
                                                           int32_t *__restrict__ inv)
{
    extern __shared__ int lds[];
    int *cnt = lds;                                   // [E]
    int *blk_ids = lds + E;                           // [PERM_TOKENS_PER_BLOCK * K]
    __shared__ int sh[16];
    const int b = blockIdx.x;
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = threadIdx.x * per, e1 = min(E, e0 + per);
    int local = 0;
    for (int e = e0; e < e1; e++)
        local += counts[e];
    int total;
    int run = block_excl_scan(local, sh, &total);
    for (int e = e0; e < e1; e++) {
        if (b == 0)
            offsets[e] = run;
        cnt[e] = run + hist[(int64_t)e * nb + b];
        run += counts[e];
    }
    if (b == 0 && threadIdx.x == 0)
        offsets[E] = total;
    const int t0 = b * PERM_TOKENS_PER_BLOCK, t1 = min(T, t0 + PERM_TOKENS_PER_BLOCK);
    for (int i = threadIdx.x; i < (t1 - t0) * K; i += blockDim.x)
        blk_ids[i] = ids[(int64_t)t0 * K + i];
    __syncthreads();
    if (threadIdx.x < WAVE) {
        const int lane = threadIdx.x;
        for (int t = t0; t < t1; t++) {
            if (lane < K) {
                const int p = t * K + lane;
                const int pos = atomicAdd(&cnt[blk_ids[p - t0 * K]], 1);
                sorted_pairs[pos] = p;
                inv[p] = pos;
            }
        }
    }
}

hipError_t launch_permute(const int32_t *ids, int T, int K, int E, int32_t *hist, int32_t *counts,
                          int32_t *offsets, int32_t *sorted_pairs, int32_t *inv, hipStream_t st)
{
    const int nb = (T + PERM_TOKENS_PER_BLOCK - 1) / PERM_TOKENS_PER_BLOCK;
    hipLaunchKernelGGL(perm_hist_kernel, dim3(nb), dim3(256), E * sizeof(int), st, ids, T, K, E, nb, hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    hipLaunchKernelGGL(perm_colscan_kernel, dim3(E), dim3(256), 0, st, hist, nb, counts);
    if ((err = hipGetLastError()) != hipSuccess)
        return err;
    const size_t lds = (E + PERM_TOKENS_PER_BLOCK * K) * sizeof(int);
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(nb), dim3(256), lds, st, ids, T, K, E, nb, hist, counts, offsets,
                       sorted_pairs, inv);
    return hipGetLastError();
}

} // namespace mxmoe
