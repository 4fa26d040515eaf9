// common.hpp -- device types, packed-layout constants and small helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace mxmoe {

constexpr int WAVE = 64;

// ---------------------------------------------------------------------------------------------
// Packed weight layouts.
//
// Every packed matrix B [N, K] (N output rows, K the reduction axis) is cut into blocks of 16 rows;
// within a row block the K axis is cut into steps. A block is laid out so that lane l of a wave
// reads bytes [16 l, 16 l + 16) and receives exactly its operand of the 16x16x32 BF16 matrix-core
// instruction: row (l % 16), inputs 8 (l / 16) .. 8 (l / 16) + 7 of each 32-wide input slice.
// MX blocks are stored row-block major: block (nb, kb) at index nb * (K / 128) + kb.
//
//  BF16 blocks: 16 rows x 32 inputs, 1024 bytes; lane l holds row l%16, inputs 8(l/16)..+7.
//               Block order: see bf16_block_index (K-chunk major).
//  MX blocks:   16 rows x 128 inputs = four 32-input slices, 1024 code bytes + 64 scale bytes.
//               Lane l's 16 code bytes are four 4-byte words; word j holds the 8 E2M1 codes of
//               row l%16, inputs 32 j + 8 (l/16) .. +7 (low nibble first). Scale byte
//               1024 + 4 n + j is the E8M0 scale of row n for slice j, so lane l reads one
//               dword at 1024 + 4 (l % 16).
// ---------------------------------------------------------------------------------------------
constexpr int BF16_BLOCK_BYTES = 1024;
constexpr int BF16_STEP = 32;
constexpr int MX_CODE_BYTES = 1024;
constexpr int MX_BLOCK_BYTES = 1088;
constexpr int MX_STEP = 128;
constexpr int TILE_HEADER_INTS = 4;   // ints before the first int4 entry of a tile list

// Dense BF16 blocks are grouped by K chunks of BF16_CHUNK_STEPS 32-wide steps (512 inputs): every
// row block's part of chunk 0, then of chunk 1, ...; within a chunk, row block by row block. Waves
// that stream one K chunk of consecutive row blocks then read one contiguous range of HBM, which
// streams far faster than ranges spread one row-block stride apart.
constexpr int BF16_CHUNK_STEPS = 16;
__host__ __device__ inline int64_t bf16_block_index(int64_t nb, int64_t kb, int64_t N, int64_t K)
{
    const int64_t ksteps = K / BF16_STEP;
    const int64_t c = kb / BF16_CHUNK_STEPS, within = kb % BF16_CHUNK_STEPS;
    const int64_t rest = ksteps - c * BF16_CHUNK_STEPS;
    const int64_t cs = rest < BF16_CHUNK_STEPS ? rest : BF16_CHUNK_STEPS;   // steps in chunk c
    return c * BF16_CHUNK_STEPS * (N / 16) + nb * cs + within;
}

__host__ __device__ inline int64_t bf16_packed_bytes(int64_t N, int64_t K) { return N * K * 2; }
__host__ __device__ inline int64_t mx_packed_bytes(int64_t N, int64_t K)
{
    return (N / 16) * (K / MX_STEP) * MX_BLOCK_BYTES;
}

// ---------------------------------------------------------------------------------------------
// Number formats.
// ---------------------------------------------------------------------------------------------
__device__ inline float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two floats -> packed BF16 bits (lo in bits 0..15), rounded to nearest even by gfx950's packed
// conversion instruction (NaN stays a quiet NaN).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// float -> BF16 bits, round to nearest even.
__device__ inline uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }

// floor(log2 |v|) of a non-zero BF16 magnitude (bits without the sign).
__device__ inline int bf16_ilogb(uint32_t mag)
{
    const uint32_t eb = mag >> 7, m = mag & 0x7Fu;
    return eb ? (int)eb - 127 : (31 - __builtin_clz(m)) - 133;
}

// E8M0 byte -> the FP32 scale 2^(e-127) of the scaled FP4 -> BF16 conversion below, in one
// instruction: 2^-127 (an FP32 denormal; kernels keep FP32 denormals) shifted by e, exact for
// e = 0..254. e = 255 gives +inf, which that conversion turns into NaN for every code (checked on
// gfx950 for all 16 codes, the same bits as a NaN scale): the E8M0 NaN.
__device__ inline float e8m0_to_f32(uint32_t e)
{
    return __builtin_amdgcn_ldexpf(__uint_as_float(0x00400000u), (int)e);
}

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) times one E8M0 scale,
// converted to eight BF16 values with gfx950's scaled FP4 -> BF16 conversion (two values per
// instruction, the byte chosen by the instruction's selector).
__device__ inline bf16x8_t mx_dequant8(uint32_t codes, float scale)
{
    union {
        bf16x2_t h[4];
        bf16x8_t v;
    } r;
    r.h[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
    r.h[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
    r.h[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
    r.h[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
    return r.v;
}

// A 16-row x 64-byte operand block (one 32-input step of 16 BF16 rows) staged in LDS with four
// consecutive lanes per row holds chunk c (16 bytes) of row r in slot 4 r + (c ^ chunk_swizzle(r)).
// The operand read (lane l: row l % 16, chunk l / 16) then hits distinct banks in every group of 8,
// 16 or 32 consecutive lanes: for a fixed chunk, the rows of each such group map to distinct slots
// modulo 8, 16 and 32. (r / 4 as the XOR repeats a slot modulo 8 within eight lanes.)
__host__ __device__ inline int chunk_swizzle(int r)
{
    return ((((r >> 2) ^ (r >> 3)) & 1) << 1) | (((r >> 1) ^ (r >> 3)) & 1);
}

__device__ inline bf16x8_t as_bf16x8(u32x4_t v)
{
    union {
        u32x4_t u;
        bf16x8_t b;
    } r;
    r.u = v;
    return r.b;
}

__device__ inline f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float silu_f32(float g) { return g / (1.0f + expf(-g)); }

__device__ inline u32x4_t load16(const void *p) { return *reinterpret_cast<const u32x4_t *>(p); }

// Weight streams are read once per call: non-temporal loads keep them from displacing the
// activations in the caches and let HBM stream at a markedly higher rate.
__device__ inline u32x4_t load16_nt(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}
__device__ inline uint32_t load4_nt(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}

// s_waitcnt immediates: at most n vector-memory operations outstanding (the other counters free),
// and no LDS (lgkm) operation outstanding (the others free).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }
constexpr int LGKM_ZERO = 15 | (7 << 4) | (0 << 8) | (3 << 14);
constexpr int vmcnt_lgkm_imm(int n) { return (n & 15) | (7 << 4) | (0 << 8) | (((n >> 4) & 3) << 14); }

// Stores into a window of `rows` rows of `ld` BF16 values that starts at `base`, through a raw
// buffer resource: a store whose byte offset lies past the window is dropped by the hardware's
// range check, so tile epilogues issue every store instruction unconditionally (the same number
// on every path, which lets the wait counts for loads issued before the stores stay exact instead
// of also waiting for the stores). rows = 0 makes every store a no-op. The last dword is the
// gfx9-family resource word (32-bit data format, no swizzle).
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ inline __amdgpu_buffer_rsrc_t row_window(void *base, int rows, int ld)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, rows * ld * 2, 0x00020000);
}
// Cache-policy argument of a non-temporal (streaming) store: outputs written once and read back only
// after far more data has passed through the caches.
constexpr int CPOL_NT = 2;
template <int CPOL = 0>
__device__ inline void store16_window(u32x4_t v, __amdgpu_buffer_rsrc_t w, int byte_offset)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v), w, byte_offset, 0, CPOL);
}

} // namespace mxmoe
