// kernels.hpp -- launch interfaces of the device kernels (internal to the library).
#pragma once

#include "common.hpp"
#include "wave.hpp"

namespace mxmoe {

enum OutKind { OUT_F32 = 0, OUT_BF16 = 1, OUT_GLU = 2 };

// Where the GEMM epilogue writes columns [col0, ...) of the logical product.
struct OutDesc {
    int kind;            // OutKind
    void *ptr;           // FP32 or BF16 row-major output
    int64_t ld;          // output row stride in elements
    int col0;            // first logical column this descriptor covers
    int n_valid;         // logical columns >= n_valid are not written (FP32 / BF16)
    const float *bias;   // FP32 only: added per logical column (nullable)
};

struct GemmArgs {
    const uint16_t *A;       // BF16 activations, row-major
    int64_t lda;             // row stride of A in elements
    const int32_t *a_index;  // nullable: product row r reads A row a_index[r] / a_div
    int a_div;
    const uint8_t *B;        // packed weights (group 0)
    int64_t b_stride;        // bytes between consecutive groups' packed weights
    int M, N, K;             // M: dense row count (ignored with a tile list)
    const int32_t *tiles;    // nullable: [0] = tile count, from element 4: int4 (group, m0, m1, -)
    int split;               // logical columns < split use `lo`, the rest `hi` ...
    int split2;              // ... and, when split2 > 0, columns >= split2 use `top`
    OutDesc lo, hi, top;
};

// Output descriptor for the columns from logical column n on. Region boundaries (split, split2)
// are multiples of the 64-column wave width, so n = a wave's first column picks one region.
__device__ inline OutDesc out_region(const GemmArgs &g, int n)
{
    return n < g.split ? g.lo : (g.split2 > 0 && n >= g.split2) ? g.top : g.hi;
}

enum GemmShape {
    GEMM_MX_GLU_M16 = 0,     // grouped MXFP4, 16 rows x one (16 gate + 16 up) pair, K over 4 waves
    GEMM_MX_M16_N64 = 1,     // grouped MXFP4 stream, 16 rows x 64 columns, one wave
    GEMM_MX_GLU_M16_N64 = 2, // grouped MXFP4, 16 rows x two (gate, up) pairs, K over 4 waves, per-step loads
};

// Tiled matrix-core product for many rows: 128 x 256 outputs per workgroup.
// Dense (g.tiles null: rows 0..M-1) or grouped (tile list, at most `max_tiles` entries).
constexpr int TILED_BM = 128;
hipError_t launch_tiled(const GemmArgs &g, bool mx, int max_tiles, hipStream_t st);
// Dense BF16 product for many rows with both operands staged through LDS (256 x 256 or 256 x 224 per
// workgroup, the narrower tile where it fills the last round of workgroups better).
bool ring_supported(const GemmArgs &g);
bool ring_preferred(const GemmArgs &g);   // supported and at least 256 tiles
hipError_t launch_ring(const GemmArgs &g, hipStream_t st);
// A-stationary grouped MXFP4 product for K <= AS_MAX_K (tile list required, BF16 output only).
constexpr int AS_MAX_K = 512;
bool astat_supported(const GemmArgs &g);
hipError_t launch_astat(const GemmArgs &g, int max_tiles, hipStream_t st);
hipError_t launch_gemm_grouped(const GemmArgs &g, GemmShape shape, int max_tiles, hipStream_t st);

// FP8 second stage: h -> MX FP8 (E4M3 codes [rows, I], E8M0 scales [rows, I/32]), and the down
// product y = bf16(h8 . Wd_e^T) over the expert tile list on MX8-packed weights (fp8.hip).
constexpr int FP8_DOWN_MAX_K = 512;
struct Fp8DownArgs {
    const uint8_t *codes;    // E4M3 h [rows, K], expert-sorted rows
    const uint8_t *scales;   // E8M0 [rows, K / 32]
    const uint8_t *B;        // MX8-packed weights of expert 0
    int64_t b_stride;        // bytes between experts
    int N, K;                // N = output columns (multiple of 64), K = I (multiple of 128, <= 512)
    const int32_t *tiles;    // expert tile list
    uint16_t *out;           // BF16 [rows, ldo]
    int64_t ldo;
};
hipError_t launch_fp8_quant(const uint16_t *h, int64_t rows, int64_t I, uint8_t *codes, uint8_t *scales,
                            hipStream_t st);
hipError_t launch_down_fp8(const Fp8DownArgs &g, bool many_rows, int max_tiles, hipStream_t st);
// A4W4 first stage: z -> MX FP4 (codes [rows, L/2], scales [rows, L/32]) and the grouped gate|up
// product with the GLU on the scaled FP4 x FP4 instruction (tile list required, N = 2I a multiple
// of 256, K a multiple of 128). Output h rows in tile-list (expert-sorted) order.
struct A4GateupArgs {
    const uint8_t *zq;          // FP4 codes of the token rows [rows, K/2]
    const uint8_t *zs;          // E8M0 scales [rows, K/32]
    const int32_t *a_index;     // row r of a tile reads token row a_index[r] / a_div
    int a_div;
    const uint8_t *B;           // A4 weight blocks, b_stride bytes per expert
    int64_t b_stride;
    int N, K;                   // 2I, Lt
    const int32_t *tiles;
    uint16_t *h;                // [P, ldh] BF16
    int ldh;
};
hipError_t launch_fp4_quant(const uint16_t *z, int64_t rows, int64_t L, uint8_t *codes, uint8_t *scales,
                            hipStream_t st);
hipError_t launch_a4_gateup(const A4GateupArgs &g, int max_tiles, hipStream_t st);
// Few rows per expert (tiles of at most 16 rows): the weight-streaming form.
hipError_t launch_a4_gateup_small(const A4GateupArgs &g, int max_tiles, hipStream_t st);
hipError_t launch_pack_gateup4(uint8_t *dst, const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                               const uint8_t *us, int64_t E, int64_t I, int64_t Lt, hipStream_t st);
hipError_t launch_pack_down8(uint8_t *dst, const uint8_t *dc, const uint8_t *ds, int64_t E, int64_t I, int64_t Lt,
                             hipStream_t st);

// Packing (moe_create) and unpacking (test hook).
hipError_t launch_pack_router(uint8_t *dst, const uint16_t *w, int64_t E, int64_t E_pad, int64_t Hin,
                              hipStream_t st);
hipError_t launch_pack_xside(uint8_t *dst, const uint16_t *wdn, const uint16_t *sg, const uint16_t *su,
                             int64_t Lt, int64_t H, int64_t S, int64_t Is, hipStream_t st);
// Router rows (zero-padded to E_pad) followed by the x-side rows, one packed [E_pad + Nx, H] matrix.
hipError_t launch_pack_router_xside(uint8_t *dst, const uint16_t *wr, int64_t E, int64_t E_pad, const uint16_t *wdn,
                                   const uint16_t *sg, const uint16_t *su, int64_t Lt, int64_t H, int64_t S, int64_t Is,
                                   hipStream_t st);
hipError_t launch_pack_outside(uint8_t *dst, const uint16_t *wup, const uint16_t *sd, int64_t Lt,
                               int64_t H, int64_t S, int64_t Is, hipStream_t st);
hipError_t launch_pack_gateup(uint8_t *dst, const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                              const uint8_t *us, int64_t E, int64_t I, int64_t Lt, hipStream_t st);
hipError_t launch_pack_down(uint8_t *dst, const uint8_t *dc, const uint8_t *ds, int64_t E, int64_t I,
                            int64_t Lt, hipStream_t st);
hipError_t launch_unpack_mx(const uint8_t *packed_expert, int64_t N, int64_t K, int interleave,
                            int which_half, uint16_t *out, hipStream_t st);

// Dense products for T <= SKINNY_MAX_M tokens: split-K FP32 partial tiles. The partials of one
// split are stored per 16-column block nb in accumulator order, SKINNY_TILE_FLOATS floats each:
// element (row, col) sits at skinny_partial_index(row, col) (rows padded to 64).
constexpr int SKINNY_MAX_M = 64;
constexpr int SKINNY_TILE_FLOATS = 4 * WAVE * 4;
__host__ __device__ inline int64_t skinny_partial_index(int row, int col)
{
    const int mf = row / 16, r = row % 16;
    const int lane = (r / 4) * 16 + col % 16;
    return (int64_t)(col / 16) * SKINNY_TILE_FLOATS + (mf * WAVE + lane) * 4 + r % 4;
}
constexpr int SKINNY_CHUNK = BF16_CHUNK_STEPS * BF16_STEP;   // K per split (one packed K chunk)
struct SkinnyArgs {
    const uint16_t *A;   // [M, lda] BF16
    int64_t lda;
    int M;
    const uint8_t *B;    // packed BF16 [N, K]
    int N, K;
    float *P;            // partials, split s at P + s * p_split_stride (>= N / 16 * SKINNY_TILE_FLOATS)
    int64_t p_split_stride;
    uint32_t *zero_word; // nullable: set to 0 by the launch (the arrival counter of the launch after it)
};
int skinny_splits(int K, int chunk_steps);
hipError_t launch_skinny(const SkinnyArgs &g, int waves, int chunk_steps, hipStream_t st);
hipError_t launch_skinny_persist(const SkinnyArgs &g, int waves, int groups, int chunk_steps, hipStream_t st);

struct XsideEpiArgs {
    const float *P;
    int64_t p_split_stride;
    int splits, M, N, Lt, shared_cols;   // N = Lt + shared_cols (2 S Is)
    uint16_t *z;                         // [M, Lt]
    uint16_t *acat;                      // [M, ldcat]; h_s written at columns Lt..
    int64_t ldcat;
    const int32_t *offsets;              // expert tile list (extra last workgroup; none if tiles is null)
    int E, bm;
    int32_t *tiles;
};
hipError_t launch_xside_epilogue(const XsideEpiArgs &e, hipStream_t st);
hipError_t launch_out_epilogue(const float *P, int64_t split_stride, int splits, int M, int N, uint16_t *out,
                               hipStream_t st);

// Routing. Logits of token t: sum over `splits` of the partials (skinny_partial_index layout) when
// `partials`, else src[t * ld + e]; plus bias[e] (nullable); written to logits_out [T, E] when
// non-null.
struct TopkArgs {
    const float *src;
    int64_t split_stride, ld;
    int splits;
    int partials;
    const float *bias;
    float *logits_out;
    int T, E, K;
    int32_t *ids;
    float *w;
    // Grouping inside the top-K launch (partials path, T <= PERM_SMALL_MAX_T): the last top-K
    // workgroup to finish writes counts / offsets / sorted_pairs / inv (and the tile list of bm rows
    // when `tiles` is set) from the ids, handed over as agent-coherent stores and an arrival counter.
    int group;
    int32_t *counts, *offsets, *sorted_pairs, *inv, *tiles;
    int bm;
    uint32_t *arrivals;   // zero when the launch starts (cleared by the product launch before it)
};
constexpr int PERM_TOKENS_PER_BLOCK = 32;
constexpr int PERM_SMALL_MAX_T = 256;
hipError_t launch_topk(const TopkArgs &a, hipStream_t st);
// Top-K from split-K partials together with the x-side epilogue (no tile lists) in one launch.
hipError_t launch_topk_xside(const TopkArgs &a, const XsideEpiArgs &e, hipStream_t st);
// Grouping for T <= PERM_SMALL_MAX_T in one workgroup; with `tiles` set it also writes the expert tile
// list of bm rows.
hipError_t launch_permute_small(const int32_t *ids, int T, int K, int E, int32_t *counts, int32_t *offsets,
                                int32_t *sorted_pairs, int32_t *inv, hipStream_t st, int bm = 0,
                                int32_t *tiles = nullptr);
// tiles (nullable): the expert tile list of bm rows, written by the scatter's first workgroup.
hipError_t launch_permute(const int32_t *ids, int T, int K, int E, int32_t *hist, int32_t *counts,
                          int32_t *offsets, int32_t *sorted_pairs, int32_t *inv, hipStream_t st, int bm,
                          int32_t *tiles);

// Forward helpers.
hipError_t launch_tilemap(const int32_t *offsets, int E, int bm, int32_t *tiles, hipStream_t st);
hipError_t launch_combine(const uint16_t *Y, int Lt, const int32_t *inv, const float *w, int T, int K,
                          uint16_t *out, int64_t ldo, hipStream_t st);

} // namespace mxmoe
