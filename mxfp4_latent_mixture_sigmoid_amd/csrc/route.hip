// route.hip -- deterministic top-K selection with sigmoid gate weights, and the grouping of
// token/expert pairs by expert (histogram, per-expert scan, stable scatter).
#include "kernels.hpp"
#include "partials.hpp"
#include "sync.hpp"


namespace mxmoe {

// Order-preserving key of a float: unsigned comparison of keys equals the float comparison, with
// -0 mapped to the key of +0 so the two compare equal. Every non-NaN value has a key > 0.
__device__ inline uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float key_value(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }

// Keys of one token, one wave: lane l holds the logits of experts l, l + 64, ... in v[]; adds the
// bias, writes logits_out (if set) and returns the order keys (0 past the last expert).
template <int SLOTS>
__device__ inline void token_keys(const TopkArgs &a, int t, float *v, uint32_t *key)
{
    const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
    for (int j = 0; j < SLOTS; j++) {
        const int e = lane + WAVE * j;
        key[j] = 0u;
        if (e < a.E) {
            if (a.bias)
                v[j] += a.bias[e];
            if (a.logits_out)
                a.logits_out[(int64_t)t * a.E + e] = v[j];
            key[j] = order_key(v[j]);
        }
    }
}

// Top-K of one token by one wave from the order keys (0 = no expert), ties to the lower expert, and
// the gate weights: sigmoid of the selected logits over their sum. Writes ids and w of token t.
// Every candidate becomes one 64-bit value, key above the complemented expert index, so the order
// (key descending, expert ascending) is plain unsigned order and all values differ.
//  1. bound: the K-th largest of the 64 lane maxima (keys only), built bit by bit from the top with
//     one ballot per bit. At least K lanes hold a key >= bound, so every selected key is >= bound.
//  2. The candidates (keys >= bound; K or a few more in practice) are gathered into `scratch` (64
//     entries of this wave); each ranks itself against all of them by lane broadcasts, and the K
//     best are placed at their ranks, so lane k then holds the rank-k expert.
//  3. With more than 64 candidates (heavy ties), K rounds of wave-wide maxima select directly.
template <int SLOTS>
__device__ inline void select_keys(const TopkArgs &a, int t, const uint32_t *key, uint64_t *scratch)
{
    const int lane = threadIdx.x & (WAVE - 1);
    const int K = a.K;
    uint64_t c[SLOTS];
    uint32_t mk = 0u;
#pragma unroll
    for (int j = 0; j < SLOTS; j++) {
        c[j] = key[j] ? ((uint64_t)key[j] << 32) | (uint32_t)~(uint32_t)(lane + WAVE * j) : 0;
        mk = key[j] > mk ? key[j] : mk;
    }
    uint32_t bound = 0u;
    for (int b = 31; b >= 0; b--) {
        const uint32_t cand = bound | (1u << b);
        if ((int)__popcll(__ballot(mk >= cand)) >= K)
            bound = cand;
    }
    int n = 0;
#pragma unroll
    for (int j = 0; j < SLOTS; j++)
        n += (key[j] != 0u && key[j] >= bound) ? 1 : 0;
    const int incl = wave_incl_scan(n);
    const int total = __shfl(incl, WAVE - 1, WAVE);
    uint32_t my_key = 0u;
    int my_id = 0;
    if (total <= WAVE) {
        int pos = incl - n;
#pragma unroll
        for (int j = 0; j < SLOTS; j++)
            if (key[j] != 0u && key[j] >= bound)
                scratch[pos++] = c[j];
        const uint64_t mine = lane < total ? scratch[lane] : 0;
        const uint32_t mh = (uint32_t)(mine >> 32), ml = (uint32_t)mine;
        int rank = 0;
        for (int m = 0; m < total; m++) {   // candidate m broadcast from its lane
            const uint32_t oh = __builtin_amdgcn_readlane(mh, m), ol = __builtin_amdgcn_readlane(ml, m);
            rank += (oh > mh || (oh == mh && ol > ml)) ? 1 : 0;
        }
        if (lane < total && rank < K)
            scratch[rank] = mine;
        const uint64_t r = lane < K ? scratch[lane] : 0;
        my_key = (uint32_t)(r >> 32);
        my_id = (int)~(uint32_t)r;
    } else {
        uint64_t left[SLOTS];
#pragma unroll
        for (int j = 0; j < SLOTS; j++)
            left[j] = c[j];
        for (int k = 0; k < K; k++) {
            uint64_t bm = left[0];
#pragma unroll
            for (int j = 1; j < SLOTS; j++)
                bm = left[j] > bm ? left[j] : bm;
            const uint32_t wk = wave_max_u32((uint32_t)(bm >> 32));
            const uint32_t wl = wave_max_u32((uint32_t)(bm >> 32) == wk ? (uint32_t)bm : 0u);
            if (lane == k) {
                my_key = wk;
                my_id = (int)~wl;
            }
            const uint64_t win = ((uint64_t)wk << 32) | wl;
#pragma unroll
            for (int j = 0; j < SLOTS; j++)
                if (left[j] == win)
                    left[j] = 0;
        }
    }
    const float s = lane < K ? 1.0f / (1.0f + expf(-key_value(my_key))) : 0.0f;
    const float sum = wave_sum_f32(s);
    if (lane < K) {
        if (a.group)   // read back by the grouping workgroup of the same launch
            store4_sc1(flat_rsrc(a.ids, (int64_t)a.T * K * 4), (int)(((int64_t)t * K + lane) * 4), (uint32_t)my_id);
        else
            a.ids[(int64_t)t * K + lane] = my_id;
        a.w[(int64_t)t * K + lane] = s / sum;
    }
}

// Grouping of the T x K pairs by expert by one workgroup (any size that is a multiple of 64), from
// ids written earlier in the same launch (agent-coherent loads). As in the one-workgroup grouping
// kernel below: a bit mask per expert marks its tokens, counts are popcounts, offsets their
// exclusive scan, and pair (t, j) goes to offsets[e] + the number of e's tokens before t.
// `lds` holds at least E * ceil(T / 32) + E + 1 words; `sh` 16 ints.
__device__ inline void group_pairs(const TopkArgs &a, uint32_t *lds, int *sh)
{
    const int T = a.T, K = a.K, E = a.E, P = T * K;
    const int W = (T + 31) / 32;
    const int nthr = (int)blockDim.x, tid = (int)threadIdx.x;
    uint32_t *masks = lds;
    int *off = reinterpret_cast<int *>(lds + E * W);
    const auto ir = flat_rsrc(a.ids, (int64_t)P * 4);
    for (int i = tid; i < E * W; i += nthr)
        masks[i] = 0u;
    __syncthreads();
    constexpr int PPT = 4;   // pairs per thread held in registers (P <= PPT * blockDim, host check)
    int ev[PPT];
#pragma unroll
    for (int u = 0; u < PPT; u++) {
        const int p = tid + u * nthr;
        ev[u] = p < P ? (int)load4_sc1(ir, p * 4) : 0;
    }
#pragma unroll
    for (int u = 0; u < PPT; u++) {
        const int p = tid + u * nthr;
        if (p < P)
            atomicOr(&masks[ev[u] * W + (p / K) / 32], 1u << ((p / K) & 31));
    }
    __syncthreads();
    const int per = (E + nthr - 1) / nthr, e0 = tid * per, e1 = min(E, e0 + per);
    int c = 0;
    for (int e = e0; e < e1; e++)
        for (int w = 0; w < W; w++)
            c += __popc(masks[e * W + w]);
    int total;
    int run = block_excl_scan(c, sh, &total);
    for (int e = e0; e < e1; e++) {
        int n = 0;
        for (int w = 0; w < W; w++)
            n += __popc(masks[e * W + w]);
        a.counts[e] = n;
        a.offsets[e] = run;
        off[e] = run;
        run += n;
    }
    if (tid == 0) {
        a.offsets[E] = total;
        off[E] = total;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PPT; u++) {
        const int p = tid + u * nthr;
        if (p >= P)
            continue;
        const int e = ev[u], t = p / K;
        const uint32_t *m = masks + e * W;
        int rank = __popc(m[t / 32] & ((1u << (t & 31)) - 1u));
        for (int w = 0; w < t / 32; w++)
            rank += __popc(m[w]);
        const int pos = off[e] + rank;
        a.sorted_pairs[pos] = p;
        a.inv[p] = pos;
    }
    if (a.tiles)
        write_tiles(off, E, a.bm, a.tiles, sh);
}

// Logits given row by row (src[t * ld + e]): one wave per token.
template <int SLOTS>
__global__ __launch_bounds__(256) void topk_kernel(const TopkArgs a)
{
    __shared__ uint64_t scratch[4][WAVE];
    const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
    const int t = blockIdx.x * 4 + wv;
    if (t >= a.T)
        return;
    float v[SLOTS];
#pragma unroll
    for (int j = 0; j < SLOTS; j++)
        v[j] = a.src[(int64_t)t * a.ld + min(lane + WAVE * j, a.E - 1)];
    uint32_t key[SLOTS];
    token_keys<SLOTS>(a, t, v, key);
    select_keys<SLOTS>(a, t, key, scratch[wv]);
}

__device__ inline int gridDim_topk(const TopkArgs &a) { return (a.T + 3) / 4; }   // top-K workgroups

// Logits as split-K partial tiles (accumulator order): eight waves per workgroup, which takes tokens
// 4 b .. 4 b + 3 (one 16-byte partial slot of an expert holds four consecutive tokens). Wave w owns
// slots j = w, w + 8 (lane l, slot j: expert l + 64 j) and adds them over all splits in split order,
// with every split's loads in flight at once; the totals go through LDS to waves 0..3, which then
// select tokens 4 b .. 4 b + 3.
template <int SLOTS>
__device__ inline void topk_wide_block(const TopkArgs &a, int blk)
{
    constexpr int WAVES = 8, SPW = (SLOTS + WAVES - 1) / WAVES;   // slots per wave
    constexpr int MAX_SPLITS = 16;
    __shared__ float red[4 * SLOTS * WAVE];                // the totals [token][slot][lane]; then the grouping's masks
    __shared__ uint64_t scratch[4][WAVE];
    __shared__ int last[1];
    __shared__ int sh[16];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const int t0 = blk * 4;
    const int mf = t0 / 16, quad = (t0 % 16) / 4;

    // expert e = lane + 64 j sits in partial tile e / 16 = lane / 16 + 4 j at column e % 16 = lane % 16
    const float *base = a.src + (int64_t)(lane / 16) * SKINNY_TILE_FLOATS + (mf * WAVE + quad * 16 + lane % 16) * 4;
    // The loads of both slots over (up to 16) splits, and the slots' bias, are all issued before any
    // is used: one memory round trip. Sums run in split order; the bias is added to the total.
    f32x4_t acc[SPW];
    float bias[SPW];
#pragma unroll
    for (int u = 0; u < SPW; u++) {
        const int j = wv + WAVES * u, e = lane + WAVE * j;
        acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        bias[u] = a.bias && j < SLOTS && e < a.E ? a.bias[e] : 0.f;
    }
    for (int s0 = 0; s0 < a.splits; s0 += MAX_SPLITS) {   // one round for up to 16 splits
        f32x4_t ld[SPW][MAX_SPLITS];
#pragma unroll
        for (int u = 0; u < SPW; u++) {
            const int j = wv + WAVES * u;
            const bool valid = j < SLOTS && lane + WAVE * j < a.E;
#pragma unroll
            for (int s = 0; s < MAX_SPLITS; s++)
                ld[u][s] = valid && s0 + s < a.splits
                               ? *reinterpret_cast<const f32x4_t *>(base + (s0 + s) * a.split_stride +
                                                                    (int64_t)j * 4 * SKINNY_TILE_FLOATS)
                               : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < SPW; u++)
#pragma unroll
            for (int s = 0; s < MAX_SPLITS; s++)
                if (s0 + s < a.splits)
                    acc[u] += ld[u][s];
    }
#pragma unroll
    for (int u = 0; u < SPW; u++) {
        const int j = wv + WAVES * u;
        if (j < SLOTS) {
            if (a.bias)
                acc[u] += f32x4_t{bias[u], bias[u], bias[u], bias[u]};
#pragma unroll
            for (int i = 0; i < 4; i++)
                red[(i * SLOTS + j) * WAVE + lane] = acc[u][i];
        }
    }
    __syncthreads();

    const int t = t0 + wv;
    if (wv < 4 && t < a.T) {
        float v[SLOTS];
#pragma unroll
        for (int j = 0; j < SLOTS; j++)
            v[j] = red[(wv * SLOTS + j) * WAVE + lane];
        uint32_t key[SLOTS];
        TopkArgs nb = a;   // the totals already hold the bias
        nb.bias = nullptr;
        token_keys<SLOTS>(nb, t, v, key);
        select_keys<SLOTS>(a, t, key, scratch[wv]);
    }
    if (!a.group)
        return;
    // The workgroup's ids stores have completed (each wave waits for its own) before one thread
    // signals; the workgroup that signals last groups every pair, reusing the totals buffer.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    asm volatile("" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
        last[0] = (int)__hip_atomic_fetch_add(a.arrivals, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  gridDim_topk(a) - 1;
    __syncthreads();
    if (last[0])
        group_pairs(a, reinterpret_cast<uint32_t *>(red), sh);
}

template <int SLOTS>
__global__ __launch_bounds__(512) void topk_wide_kernel(const TopkArgs a)
{
    topk_wide_block<SLOTS>(a, blockIdx.x);
}

// One launch for two independent consumers of the combined router + x-side partials: workgroups
// 0 .. ntopk-1 select the top-K of four tokens each, the rest run the x-side epilogue (512 items
// per workgroup), so the two overlap instead of running back to back.
template <int SLOTS>
__global__ __launch_bounds__(512) void topk_xside_kernel(const TopkArgs a, const XsideEpiArgs e, int ntopk)
{
    if ((int)blockIdx.x < ntopk)
        topk_wide_block<SLOTS>(a, blockIdx.x);
    else
        xside_epi_item(e, (int64_t)(blockIdx.x - ntopk) * blockDim.x + threadIdx.x);
}

static bool group_args_ok(const TopkArgs &a)
{
    if (!a.group)
        return true;
    // the masks (E x ceil(T / 32) words) and offsets (E + 1) reuse the top-K reduction buffer of at
    // least 64 E bytes, which holds them for T <= SKINNY_MAX_M
    return a.arrivals && a.counts && a.offsets && a.sorted_pairs && a.inv && a.T <= SKINNY_MAX_M &&
           (int64_t)a.T * a.K <= 4 * 512 && (!a.tiles || a.bm >= 1);
}

hipError_t launch_topk_xside(const TopkArgs &a, const XsideEpiArgs &e, hipStream_t st)
{
    if (!a.partials || a.T > SKINNY_MAX_M || a.K > WAVE || a.E > 16 * WAVE || e.tiles || !group_args_ok(a))
        return hipErrorInvalidValue;
    const int ntopk = (a.T + 3) / 4;
    const int64_t items = (int64_t)(e.Lt / 16 + e.shared_cols / 32) * 4 * WAVE;
    const dim3 grid(ntopk + (unsigned)((items + 511) / 512));
    const int slots = (a.E + WAVE - 1) / WAVE;
    if (slots <= 4)
        hipLaunchKernelGGL(topk_xside_kernel<4>, grid, dim3(512), 0, st, a, e, ntopk);
    else if (slots <= 8)
        hipLaunchKernelGGL(topk_xside_kernel<8>, grid, dim3(512), 0, st, a, e, ntopk);
    else
        hipLaunchKernelGGL(topk_xside_kernel<16>, grid, dim3(512), 0, st, a, e, ntopk);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t st)
{
    const dim3 grid((a.T + 3) / 4);
    if (a.K > WAVE || a.E > 16 * WAVE || (a.partials && a.T > SKINNY_MAX_M) || (a.group && !a.partials) ||
        !group_args_ok(a))
        return hipErrorInvalidValue;
    const int slots = (a.E + WAVE - 1) / WAVE;
    if (a.partials) {
        if (slots <= 4)
            hipLaunchKernelGGL(topk_wide_kernel<4>, grid, dim3(512), 0, st, a);
        else if (slots <= 8)
            hipLaunchKernelGGL(topk_wide_kernel<8>, grid, dim3(512), 0, st, a);
        else
            hipLaunchKernelGGL(topk_wide_kernel<16>, grid, dim3(512), 0, st, a);
    } else if (slots <= 2) {
        hipLaunchKernelGGL(topk_kernel<2>, grid, dim3(256), 0, st, a);
    } else {
        hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

// Grouping by expert for T <= 256 tokens in one workgroup: a bit mask per expert marks the tokens
// routed to it (the K experts of a token are distinct, so each (token, expert) bit is set once);
// counts are popcounts, offsets their exclusive scan, and the position of pair (t, j) is
// offsets[e] + the number of tokens before t in e's mask -- stable, with no ordering races.
// With `tiles` set, the workgroup also writes the expert tile list(s) of `bm` rows from the offsets.
__global__ __launch_bounds__(1024) void perm_small_kernel(const int32_t *__restrict__ ids, int T, int K, int E,
                                                          int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                          int32_t *__restrict__ sorted_pairs, int32_t *__restrict__ inv,
                                                          int bm, int32_t *__restrict__ tiles)
{
    extern __shared__ uint32_t masks[];               // [E][W] then off[E + 1]
    __shared__ int sh[16];
    const int W = (T + 31) / 32;
    int *off = reinterpret_cast<int *>(masks + E * W);
    for (int i = threadIdx.x; i < E * W; i += blockDim.x)
        masks[i] = 0u;
    __syncthreads();
    const int P = T * K;
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const int t = p / K;
        atomicOr(&masks[ids[p] * W + t / 32], 1u << (t & 31));
    }
    __syncthreads();
    int c = 0;
    if ((int)threadIdx.x < E)
        for (int w = 0; w < W; w++)
            c += __popc(masks[threadIdx.x * W + w]);
    int total;
    const int ex = block_excl_scan(c, sh, &total);
    if ((int)threadIdx.x < E) {
        counts[threadIdx.x] = c;
        offsets[threadIdx.x] = ex;
        off[threadIdx.x] = ex;
    }
    if (threadIdx.x == 0) {
        offsets[E] = total;
        off[E] = total;
    }
    __syncthreads();
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const int t = p / K, e = ids[p];
        const uint32_t *m = masks + e * W;
        int rank = __popc(m[t / 32] & ((1u << (t & 31)) - 1u));
        for (int w = 0; w < t / 32; w++)
            rank += __popc(m[w]);
        const int pos = off[e] + rank;
        sorted_pairs[pos] = p;
        inv[p] = pos;
    }
    if (tiles)
        write_tiles(off, E, bm, tiles, sh);
}

hipError_t launch_permute_small(const int32_t *ids, int T, int K, int E, int32_t *counts, int32_t *offsets,
                                int32_t *sorted_pairs, int32_t *inv, hipStream_t st, int bm, int32_t *tiles)
{
    if (T > PERM_SMALL_MAX_T || E > 1024 || (tiles && bm < 1))
        return hipErrorInvalidValue;
    const size_t lds = ((size_t)E * ((T + 31) / 32) + E + 1) * sizeof(uint32_t);
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(1024), lds, st, ids, T, K, E, counts, offsets, sorted_pairs,
                       inv, bm, tiles);
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
// LDS counters and every pair lands at offsets[e] + (pairs of e in earlier tokens). Every block
// computes all the offsets; block 0 also writes them, and the expert tile list of bm rows when
// `tiles` is set.
__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t *__restrict__ ids, int T, int K, int E,
                                                           int nb, const int32_t *__restrict__ hist,
                                                           const int32_t *__restrict__ counts,
                                                           int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ sorted_pairs,
                                                           int32_t *__restrict__ inv, int bm,
                                                           int32_t *__restrict__ tiles)
{
    extern __shared__ int lds[];
    int *cnt = lds;                                   // [E]
    int *blk_ids = lds + E;                           // [PERM_TOKENS_PER_BLOCK * K]
    int *off = blk_ids + PERM_TOKENS_PER_BLOCK * K;   // [E + 1], block 0 with a tile list only
    __shared__ int sh[16];
    const int b = blockIdx.x;
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = threadIdx.x * per, e1 = min(E, e0 + per);
    int local = 0;
    for (int e = e0; e < e1; e++)
        local += counts[e];
    int total;
    int run = block_excl_scan(local, sh, &total);
    const bool list = b == 0 && tiles;
    for (int e = e0; e < e1; e++) {
        if (b == 0)
            offsets[e] = run;
        if (list)
            off[e] = run;
        cnt[e] = run + hist[(int64_t)e * nb + b];
        run += counts[e];
    }
    if (b == 0 && threadIdx.x == 0) {
        offsets[E] = total;
        if (list)
            off[E] = total;
    }
    if (list) {   // block-uniform: every thread of block 0 takes part
        __syncthreads();
        write_tiles(off, E, bm, tiles, sh);
    }
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
                          int32_t *offsets, int32_t *sorted_pairs, int32_t *inv, hipStream_t st, int bm,
                          int32_t *tiles)
{
    const int nb = (T + PERM_TOKENS_PER_BLOCK - 1) / PERM_TOKENS_PER_BLOCK;
    hipLaunchKernelGGL(perm_hist_kernel, dim3(nb), dim3(256), E * sizeof(int), st, ids, T, K, E, nb, hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    hipLaunchKernelGGL(perm_colscan_kernel, dim3(E), dim3(256), 0, st, hist, nb, counts);
    if ((err = hipGetLastError()) != hipSuccess)
        return err;
    if (tiles && bm <= 0)
        return hipErrorInvalidValue;
    const size_t lds = (E + PERM_TOKENS_PER_BLOCK * K + (tiles ? E + 1 : 0)) * sizeof(int);
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(nb), dim3(256), lds, st, ids, T, K, E, nb, hist, counts, offsets,
                       sorted_pairs, inv, bm, tiles);
    return hipGetLastError();
}

} // namespace mxmoe
