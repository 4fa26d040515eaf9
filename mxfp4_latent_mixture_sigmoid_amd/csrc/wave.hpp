// wave.hpp -- wave- and workgroup-level reductions and scans (DPP cross-lane moves), and the
// expert tile-list builder shared by the kernels that produce it.
#pragma once

#include "common.hpp"

namespace mxmoe {

// DPP controls (GFX9 encoding).
constexpr int DPP_QUAD_1032 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_ROR4 = 0x124;
constexpr int DPP_ROW_ROR8 = 0x128;
constexpr int DPP_ROW_BCAST15 = 0x142;
constexpr int DPP_ROW_BCAST31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ inline uint32_t dpp_u32(uint32_t old, uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Maximum / minimum over the 64 lanes, returned to every lane (wave-uniform).
__device__ inline uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<DPP_QUAD_1032, 0xF>(v, v));
    v = max(v, dpp_u32<DPP_QUAD_2301, 0xF>(v, v));
    v = max(v, dpp_u32<DPP_ROW_ROR4, 0xF>(v, v));
    v = max(v, dpp_u32<DPP_ROW_ROR8, 0xF>(v, v));
    v = max(v, dpp_u32<DPP_ROW_BCAST15, 0xA>(v, v));
    v = max(v, dpp_u32<DPP_ROW_BCAST31, 0xC>(v, v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ inline uint32_t wave_min_u32(uint32_t v)
{
    v = min(v, dpp_u32<DPP_QUAD_1032, 0xF>(v, v));
    v = min(v, dpp_u32<DPP_QUAD_2301, 0xF>(v, v));
    v = min(v, dpp_u32<DPP_ROW_ROR4, 0xF>(v, v));
    v = min(v, dpp_u32<DPP_ROW_ROR8, 0xF>(v, v));
    v = min(v, dpp_u32<DPP_ROW_BCAST15, 0xA>(v, v));
    v = min(v, dpp_u32<DPP_ROW_BCAST31, 0xC>(v, v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Float sum over the 64 lanes in a fixed combination order, identical in every lane.
__device__ inline float wave_sum_f32(float x)
{
    uint32_t v = __float_as_uint(x);
    v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<DPP_QUAD_1032, 0xF>(0u, v)));
    v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<DPP_QUAD_2301, 0xF>(0u, v)));
    v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<DPP_ROW_ROR4, 0xF>(0u, v)));
    v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<DPP_ROW_ROR8, 0xF>(0u, v)));
    v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<DPP_ROW_BCAST15, 0xA>(0u, v)));
    v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<DPP_ROW_BCAST31, 0xC>(0u, v)));
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)v, 63));
}

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

// Exclusive prefix sum of one value per thread over the workgroup (blockDim <= 1024); every
// thread must call it. `sh` holds >= 16 ints of LDS; *total receives the workgroup sum.
__device__ inline int block_excl_scan(int v, int *sh, int *total)
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

// Expert tile list for row tiles of `bm` rows (every thread of the block calls it; thread i takes
// the run of consecutive experts i*per .. i*per+per-1, per = ceil(E / blockDim)). Expert e with n_e
// rows gets ceil(n_e / bm) tiles of consecutive rows of the expert-sorted order, listed expert by
// expert. Layout: tiles[0] = tile count, then from element TILE_HEADER_INTS one int4 (expert,
// first row, end row, 0) per tile.
__device__ inline void write_tiles(const int32_t *offsets, int E, int bm, int32_t *tiles, int *sh)
{
    const int per = (E + (int)blockDim.x - 1) / (int)blockDim.x;
    const int e0 = (int)threadIdx.x * per;
    int c = 0;
    for (int i = 0; i < per; i++) {
        const int e = e0 + i;
        if (e < E)
            c += (offsets[e + 1] - offsets[e] + bm - 1) / bm;
    }
    int total;
    int base = block_excl_scan(c, sh, &total);
    int4 *out = reinterpret_cast<int4 *>(tiles + TILE_HEADER_INTS);
    for (int i = 0; i < per; i++) {
        const int e = e0 + i;
        if (e >= E)
            break;
        const int beg = offsets[e], n = offsets[e + 1] - beg;
        for (int j = 0; j * bm < n; j++)
            out[base++] = int4{e, beg + j * bm, min(beg + (j + 1) * bm, beg + n), 0};
    }
    if (threadIdx.x == 0)
        tiles[0] = total;
}

} // namespace mxmoe
