// Device-side helpers shared by the gfx950 kernels of libsmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smoe {

constexpr int kMaxExperts = 16;

struct QPtr {
    const uint8_t *codes;
    const void *scales;   // f32, or f16 when the launch says scale_bytes == 2
};

// Zero point of a b-bit affine code: 7.5 at 4 bits, 1.5 at 2 bits (Metal Compute
// Kernels, "Fused FFN Kernels -- One Simdgroup Per Output Row").
template <int BITS>
struct QFormat {
    static constexpr int kCodesPerChunk = 128 / BITS;   // codes in one 16-byte chunk
    static constexpr float kZ = BITS == 4 ? 7.5f : 1.5f;
    static constexpr float kInvZ = 1.0f / kZ;
};

// Makes the bits of v unknown to the optimiser.  Without it the compiler folds
// "mask the nibbles, then take byte p" into one AND per code; with it each masked
// dword feeds four v_cvt_f32_ubyteN conversions directly.
__device__ __forceinline__ uint32_t opaque(uint32_t v)
{
    asm("" : "+v"(v));
    return v;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of W lanes (W a power of two <= 64); every lane of a
// group receives the group's sum.  Within a 16-lane DPP row: swap neighbours,
// swap pairs, mirror halves of 8, mirror halves of 16.
template <int W>
__device__ __forceinline__ float lane_group_sum(float v)
{
    if constexpr (W >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (W >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v += dpp<0x141>(v);   // row_half_mirror
    if constexpr (W >= 16) v += dpp<0x140>(v);  // row_mirror
    if constexpr (W >= 32) v += __shfl_xor(v, 16);
    if constexpr (W >= 64) v += __shfl_xor(v, 32);
    return v;
}

__device__ __forceinline__ uint4 load16(const uint8_t *p)
{
    return *reinterpret_cast<const uint4 *>(p);
}

__device__ __forceinline__ float silu(float t)
{
    return t / (1.0f + expf(-t));
}

}  // namespace smoe
