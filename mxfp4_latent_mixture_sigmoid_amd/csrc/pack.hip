// pack.hip -- one-time packing of canonical weights into matrix-core fragment order, and the
// test-hook unpacking of MXFP4 experts back to BF16 through the GEMMs' dequantisation.
#include "kernels.hpp"

namespace mxmoe {

// One thread writes one lane's 16 bytes of one 16x32 BF16 block of a logical matrix [N, K].
// The logical row/column is mapped to its canonical source by `fetch`.
template <typename Fetch>
__global__ void pack_bf16_kernel(uint8_t *__restrict__ dst, int64_t N, int64_t K, Fetch fetch)
{
    const int64_t chunk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t kblocks = K / BF16_STEP;
    if (chunk >= (N / 16) * kblocks * WAVE)
        return;
    const int lane = (int)(chunk % WAVE);
    const int64_t blk = chunk / WAVE;
    const int64_t nb = blk / kblocks, kb = blk % kblocks;
    const int64_t n = nb * 16 + (lane & 15);
    const int64_t k = kb * BF16_STEP + 8 * (lane >> 4);
    *reinterpret_cast<u32x4_t *>(dst + bf16_block_index(nb, kb, N, K) * BF16_BLOCK_BYTES + lane * 16) = fetch(n, k);
}

struct FetchRouter {          // [E_pad, Hin]: router rows, zero rows past E
    const uint16_t *w;
    int64_t E, Hin;
    __device__ u32x4_t operator()(int64_t n, int64_t k) const
    {
        if (n >= E)
            return u32x4_t{0, 0, 0, 0};
        return load16(w + n * Hin + k);
    }
};

struct FetchXside {           // [Lt + 2 S Is, H]: down-projection rows, then per shared expert
    const uint16_t *wdn, *sg, *su;   // 16 gate rows / 16 up rows alternating
    int64_t Lt, H, Is;
    __device__ u32x4_t operator()(int64_t n, int64_t k) const
    {
        if (n < Lt)
            return load16(wdn + n * H + k);
        const int64_t r = n - Lt, s = r / (2 * Is), q = r % (2 * Is);
        const int64_t j = (q / 32) * 16 + (q % 16);
        const uint16_t *src = (q % 32) < 16 ? sg : su;
        return load16(src + (s * Is + j) * H + k);
    }
};

struct FetchRouterXside {     // [E_pad + Lt + 2 S Is, H]: router rows (zero past E), then the x-side rows
    FetchRouter r;
    FetchXside x;
    int64_t E_pad;
    __device__ u32x4_t operator()(int64_t n, int64_t k) const { return n < E_pad ? r(n, k) : x(n - E_pad, k); }
};

struct FetchOutside {         // [H, Lt + S Is]: up-projection row n, then shared down rows n
    const uint16_t *wup, *sd;
    int64_t Lt, H, Is;
    __device__ u32x4_t operator()(int64_t n, int64_t k) const
    {
        if (k < Lt)
            return load16(wup + n * Lt + k);
        const int64_t c = k - Lt, s = c / Is, j = c % Is;
        return load16(sd + (s * H + n) * Is + j);
    }
};

// Logical MX row -> canonical (matrix, row). Gate/up matrices are interleaved per 16 rows.
struct MxRows {
    const uint8_t *codes[2], *scales[2];  // [0] gate or down, [1] up (gate/up only)
    int64_t rows;                         // canonical rows per expert
    int interleave;                       // 1: logical row n -> gate/up by 16-row halves
    __device__ void map(int64_t n, int &m, int64_t &row) const
    {
        if (interleave) {
            m = (int)((n % 32) >= 16);
            row = (n / 32) * 16 + (n % 16);
        } else {
            m = 0;
            row = n;
        }
    }
};

// One thread writes one lane's 16 code bytes (and, for lanes < 16, one dword of scales) of one
// 16x128 MX block of expert e's logical matrix [N, K].
__global__ void pack_mx_kernel(uint8_t *__restrict__ dst, int64_t E, int64_t N, int64_t K, MxRows src)
{
    const int64_t chunk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t kblocks = K / MX_STEP, nblocks = N / 16;
    if (chunk >= E * nblocks * kblocks * WAVE)
        return;
    const int lane = (int)(chunk % WAVE);
    const int64_t blk = chunk / WAVE;                 // = (e * nblocks + nb) * kblocks + kb
    const int64_t e = blk / (nblocks * kblocks);
    const int64_t nb = (blk / kblocks) % nblocks, kb = blk % kblocks;
    int m;
    int64_t row;
    const int64_t n = nb * 16 + (lane & 15);
    src.map(n, m, row);
    const uint8_t *codes = src.codes[m] + (e * src.rows + row) * (K / 2);
    const uint8_t *scales = src.scales[m] + (e * src.rows + row) * (K / 32);
    u32x4_t v;
    for (int j = 0; j < 4; j++) {
        const int64_t k = kb * MX_STEP + 32 * j + 8 * (lane >> 4);
        v[j] = *reinterpret_cast<const uint32_t *>(codes + k / 2);
    }
    uint8_t *out = dst + blk * MX_BLOCK_BYTES;
    *reinterpret_cast<u32x4_t *>(out + lane * 16) = v;
    if (lane < 16) {
        uint32_t s = 0;
        for (int j = 0; j < 4; j++)
            s |= (uint32_t)scales[kb * 4 + j] << (8 * j);
        *reinterpret_cast<uint32_t *>(out + MX_CODE_BYTES + 4 * lane) = s;
    }
}

// Inverse of pack_mx_kernel for one expert and one canonical matrix, dequantised to BF16.
__global__ void unpack_mx_kernel(const uint8_t *__restrict__ packed, int64_t N, int64_t K,
                                 int interleave, int which_half, uint16_t *__restrict__ out)
{
    const int64_t chunk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t kblocks = K / MX_STEP, nblocks = N / 16;
    if (chunk >= nblocks * kblocks * WAVE)
        return;
    const int lane = (int)(chunk % WAVE);
    const int64_t blk = chunk / WAVE;
    const int64_t nb = blk / kblocks, kb = blk % kblocks;
    const int64_t n = nb * 16 + (lane & 15);
    int64_t row = n;
    if (interleave) {
        if ((int)((n % 32) >= 16) != which_half)
            return;
        row = (n / 32) * 16 + (n % 16);
    }
    const uint8_t *b = packed + blk * MX_BLOCK_BYTES;
    const u32x4_t codes = load16(b + lane * 16);
    const uint32_t sc = *reinterpret_cast<const uint32_t *>(b + MX_CODE_BYTES + 4 * (lane & 15));
    for (int j = 0; j < 4; j++) {
        const bf16x8_t v = mx_dequant8(codes[j], e8m0_to_f32((sc >> (8 * j)) & 0xFFu));
        const int64_t k = kb * MX_STEP + 32 * j + 8 * (lane >> 4);
        union {
            bf16x8_t b;
            u32x4_t u;
        } cv;
        cv.b = v;
        *reinterpret_cast<u32x4_t *>(out + row * K + k) = cv.u;
    }
}

static inline unsigned grid_for(int64_t threads, int block) { return (unsigned)((threads + block - 1) / block); }

hipError_t launch_pack_router(uint8_t *dst, const uint16_t *w, int64_t E, int64_t E_pad, int64_t Hin,
                              hipStream_t st)
{
    const int64_t thr = (E_pad / 16) * (Hin / BF16_STEP) * WAVE;
    hipLaunchKernelGGL(pack_bf16_kernel<FetchRouter>, dim3(grid_for(thr, 256)), dim3(256), 0, st, dst,
                       E_pad, Hin, FetchRouter{w, E, Hin});
    return hipGetLastError();
}

hipError_t launch_pack_xside(uint8_t *dst, const uint16_t *wdn, const uint16_t *sg, const uint16_t *su,
                             int64_t Lt, int64_t H, int64_t S, int64_t Is, hipStream_t st)
{
    const int64_t N = Lt + 2 * S * Is;
    const int64_t thr = (N / 16) * (H / BF16_STEP) * WAVE;
    hipLaunchKernelGGL(pack_bf16_kernel<FetchXside>, dim3(grid_for(thr, 256)), dim3(256), 0, st, dst, N,
                       H, FetchXside{wdn, sg, su, Lt, H, Is});
    return hipGetLastError();
}

hipError_t launch_pack_router_xside(uint8_t *dst, const uint16_t *wr, int64_t E, int64_t E_pad, const uint16_t *wdn,
                                   const uint16_t *sg, const uint16_t *su, int64_t Lt, int64_t H, int64_t S, int64_t Is,
                                   hipStream_t st)
{
    const int64_t N = E_pad + Lt + 2 * S * Is;
    const int64_t thr = (N / 16) * (H / BF16_STEP) * WAVE;
    hipLaunchKernelGGL(pack_bf16_kernel<FetchRouterXside>, dim3(grid_for(thr, 256)), dim3(256), 0, st, dst, N, H,
                       FetchRouterXside{FetchRouter{wr, E, H}, FetchXside{wdn, sg, su, Lt, H, Is}, E_pad});
    return hipGetLastError();
}

hipError_t launch_pack_outside(uint8_t *dst, const uint16_t *wup, const uint16_t *sd, int64_t Lt,
                               int64_t H, int64_t S, int64_t Is, hipStream_t st)
{
    const int64_t K = Lt + S * Is;
    const int64_t thr = (H / 16) * (K / BF16_STEP) * WAVE;
    hipLaunchKernelGGL(pack_bf16_kernel<FetchOutside>, dim3(grid_for(thr, 256)), dim3(256), 0, st, dst, H,
                       K, FetchOutside{wup, sd, Lt, H, Is});
    return hipGetLastError();
}

hipError_t launch_pack_gateup(uint8_t *dst, const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                              const uint8_t *us, int64_t E, int64_t I, int64_t Lt, hipStream_t st)
{
    MxRows src{{gc, uc}, {gs, us}, I, 1};
    const int64_t thr = E * (2 * I / 16) * (Lt / MX_STEP) * WAVE;
    hipLaunchKernelGGL(pack_mx_kernel, dim3(grid_for(thr, 256)), dim3(256), 0, st, dst, E, 2 * I, Lt, src);
    return hipGetLastError();
}

hipError_t launch_pack_down(uint8_t *dst, const uint8_t *dc, const uint8_t *ds, int64_t E, int64_t I,
                            int64_t Lt, hipStream_t st)
{
    MxRows src{{dc, dc}, {ds, ds}, Lt, 0};
    const int64_t thr = E * (Lt / 16) * (I / MX_STEP) * WAVE;
    hipLaunchKernelGGL(pack_mx_kernel, dim3(grid_for(thr, 256)), dim3(256), 0, st, dst, E, Lt, I, src);
    return hipGetLastError();
}

hipError_t launch_unpack_mx(const uint8_t *packed_expert, int64_t N, int64_t K, int interleave,
                            int which_half, uint16_t *out, hipStream_t st)
{
    const int64_t thr = (N / 16) * (K / MX_STEP) * WAVE;
    hipLaunchKernelGGL(unpack_mx_kernel, dim3(grid_for(thr, 256)), dim3(256), 0, st, packed_expert, N, K,
                       interleave, which_half, out);
    return hipGetLastError();
}

} // namespace mxmoe
