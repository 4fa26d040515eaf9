// sync.hpp -- hand-offs between workgroups of one kernel without cache write-back fences.
//
// On gfx950 each XCD has its own L2; the memory model's agent-scope release fence writes back the
// whole L2 (buffer_wbl2) and the acquire fence invalidates it, which costs far more than the data
// being handed over (measured: one release per 16 KB streamed unit made a 24 us product take
// 274 us). Data that one workgroup hands to another inside a kernel therefore travels as
// agent-coherent accesses instead -- stores and loads with the sc1 cache policy, the same
// instructions the compiler emits for agent-scope relaxed atomic stores and loads -- and the
// writer waits for its stores to complete (s_waitcnt) before it signals on a counter; the reader
// issues its loads only after its counter access has returned. A counter is a plain 32-bit word
// that the launch before the one using it sets to zero, so a kernel boundary orders the clearing
// before every arrival and no workspace clearing launch is needed.
#pragma once

#include "common.hpp"

namespace mxmoe {

constexpr int CPOL_SC1 = 16;   // agent-coherent access (sc1)

// Raw buffer resource over [base, base + bytes) (bytes < 2^31).
__device__ inline __amdgpu_buffer_rsrc_t flat_rsrc(const void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline void store16_sc1(__amdgpu_buffer_rsrc_t r, int byte_offset, f32x4_t v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v), r, byte_offset, 0, CPOL_SC1);
}

__device__ inline f32x4_t load16_sc1(__amdgpu_buffer_rsrc_t r, int byte_offset)
{
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, CPOL_SC1));
}

__device__ inline void store4_sc1(__amdgpu_buffer_rsrc_t r, int byte_offset, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32((int)v, r, byte_offset, 0, CPOL_SC1);
}

__device__ inline uint32_t load4_sc1(__amdgpu_buffer_rsrc_t r, int byte_offset)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, byte_offset, 0, CPOL_SC1);
}

} // namespace mxmoe
