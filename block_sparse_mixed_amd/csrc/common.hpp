// Device helpers shared by the kernels: geometry of a block, E8M0 scale
// exponents, and packing through the gfx950 conversion instructions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <tuple>
#include <utility>

#include "da2_internal.hpp"

namespace da2 {

// Launch a kernel and return the error of this launch alone. (The "last
// error" of the runtime also holds failures of unrelated earlier calls made
// by other code in the process, so it is not consulted.)
template <typename... P, typename... A>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                         A&&... args) {
    std::tuple<P...> vals(std::forward<A>(args)...);
    return std::apply(
        [&](auto&... v) {
            void* ptrs[] = {static_cast<void*>(&v)...};
            return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem, stream);
        },
        vals);
}

// Window (block) position of block index blk: (frame, window row, window column).
struct BlockPos {
    int t, wy, wx;
};

__device__ __forceinline__ BlockPos block_pos(const Geo& g, int blk) {
    const int per_frame = g.n_wy * g.n_wx;
    BlockPos p;
    p.t = blk / per_frame;
    const int r = blk - p.t * per_frame;
    p.wy = r / g.n_wx;
    p.wx = r - p.wy * g.n_wx;
    return p;
}

// Raster index of slot s of block p, or -1 for a padded slot. Slots are
// row-major inside the window.
__device__ __forceinline__ int64_t slot_raster(const Geo& g, const BlockPos& p, int s) {
    if (s >= g.block_size) return -1;
    const int iy = s / g.win_w;
    const int ix = s - iy * g.win_w;
    const int y = p.wy * g.win_h + iy;
    const int x = p.wx * g.win_w + ix;
    if (y >= g.grid_h || x >= g.grid_w) return -1;
    return ((int64_t)p.t * g.grid_h + y) * g.grid_w + x;
}

// Number of real tokens in block p.
__device__ __forceinline__ int block_count(const Geo& g, const BlockPos& p) {
    const int rows = min(g.win_h, g.grid_h - p.wy * g.win_h);
    const int cols = min(g.win_w, g.grid_w - p.wx * g.win_w);
    return rows * cols;
}

// Smallest integer e with amax <= F * 2^e, F = 1.m_F * 2^E_F, clamped to
// [-127, 127]; amax is a non-negative fp32 magnitude (0 gives -127). With
// amax = M * 2^E, M in [1, 2): e = E - E_F + (M > m_F). Subnormal amax only
// arises for amax < 2^-126, where the clamp decides anyway.
template <int kEF, uint32_t kMantF>
__device__ __forceinline__ int scale_exponent(float amax) {
    const uint32_t b = __float_as_uint(amax);
    const int ef = (int)((b >> 23) & 0xFF);
    if (ef == 0) return -127;
    const int e = ef - 127 - kEF + (((b & 0x7FFFFFu) > kMantF) ? 1 : 0);
    return min(127, max(-127, e));
}
// E4M3: F = 448 = 1.75 * 2^8; E2M1: F = 6 = 1.5 * 2^2.
__device__ __forceinline__ int fp8_exponent(float amax) { return scale_exponent<8, 0x600000u>(amax); }
__device__ __forceinline__ int fp4_exponent(float amax) { return scale_exponent<2, 0x400000u>(amax); }

// 2^k for an integer k in [-126, 127], exactly.
__device__ __forceinline__ float exp2i(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Four values -> four E4M3 codes (round to nearest even), packed low byte first.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
    // the first conversion writes the low half and keeps the high half of
    // its "old" operand, which the second conversion overwrites: any old
    // value will do, and reusing a's register saves a move
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Two E4M3 codes (bytes 0-1, or 2-3 when hi) -> two bf16 values, packed low
// first. Exact: an E4M3 value has at most 4 significant bits.
template <bool kHi>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t codes) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    const v2f f = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, kHi);
    return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u);
}

// Eight values -> eight E2M1 codes (round to nearest even, saturating at 6),
// packed low nibble first.
__device__ __forceinline__ uint32_t pack_fp4x8(const float* v) {
    // every byte is written below, so the "old" operand is irrelevant
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(__float_as_uint(v[0]), v[0], v[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
    return w;
}

}  // namespace da2
