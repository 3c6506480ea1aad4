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

// Position of block blk. Window layout: every block is one window, numbered
// (frame, window row, window column). Packed layout: the full windows come
// first, numbered the same way among themselves, then blocks cut from one
// stream of the partial windows' tokens (window by window in (frame, window
// row, window column) order, row-major inside each window); for those,
// edge0 is the stream position of slot 0 (-1 for a window block).
struct BlockPos {
    int t, wy, wx;
    int edge0;
};

__host__ __device__ __forceinline__ BlockPos block_pos(const Geo& g, int blk) {
    BlockPos p;
    p.edge0 = -1;
    if (g.pack && blk >= g.n_full) {
        p.t = p.wy = p.wx = 0;
        p.edge0 = (blk - g.n_full) * g.block_size;
        return p;
    }
    const int nwy = g.pack ? g.fwy : g.n_wy;
    const int nwx = g.pack ? g.fwx : g.n_wx;
    const int per_frame = nwy * nwx;
    p.t = blk / per_frame;
    const int r = blk - p.t * per_frame;
    p.wy = r / nwx;
    p.wx = r - p.wy * nwx;
    return p;
}

// Raster index of slot s of block p, or -1 for a padded slot. Slots are
// row-major inside a window. In the packed stream, a frame's partial windows
// are the right-hand column (window rows 0 .. fwy-1, rem_w columns wide)
// followed by the bottom row (rem_h rows high, every window column).
__host__ __device__ __forceinline__ int64_t slot_raster(const Geo& g, const BlockPos& p, int s) {
    if (s >= g.block_size) return -1;
    int t, y, x;
    if (p.edge0 >= 0) {
        const int e = p.edge0 + s;
        if (e >= g.edge_total) return -1;
        t = e / g.edge_frame;
        const int r = e - t * g.edge_frame;
        const int rem_w = g.grid_w - g.fwx * g.win_w;
        const int right = g.fwy * g.win_h * rem_w;          // tokens of the right-hand column
        if (r < right) {                                     // (rem_w > 0 here)
            const int wsz = g.win_h * rem_w;
            const int wy = r / wsz;
            const int r2 = r - wy * wsz;
            const int iy = r2 / rem_w;
            y = wy * g.win_h + iy;
            x = g.fwx * g.win_w + (r2 - iy * rem_w);
        } else {                                             // (rem_h > 0 here)
            const int rem_h = g.grid_h - g.fwy * g.win_h;
            const int r1 = r - right;
            const int wx = r1 / (rem_h * g.win_w);
            const int r2 = r1 - wx * rem_h * g.win_w;
            const int ww = g.grid_w - wx * g.win_w < g.win_w ? g.grid_w - wx * g.win_w : g.win_w;
            const int iy = r2 / ww;
            y = g.fwy * g.win_h + iy;
            x = wx * g.win_w + (r2 - iy * ww);
        }
    } else {
        const int iy = s / g.win_w;
        const int ix = s - iy * g.win_w;
        t = p.t;
        y = p.wy * g.win_h + iy;
        x = p.wx * g.win_w + ix;
        if (y >= g.grid_h || x >= g.grid_w) return -1;
    }
    return ((int64_t)t * g.grid_h + y) * g.grid_w + x;
}

// Number of real tokens in block p.
__host__ __device__ __forceinline__ int block_count(const Geo& g, const BlockPos& p) {
    if (p.edge0 >= 0) return g.edge_total - p.edge0 < g.block_size ? g.edge_total - p.edge0 : g.block_size;
    const int rows = g.grid_h - p.wy * g.win_h < g.win_h ? g.grid_h - p.wy * g.win_h : g.win_h;
    const int cols = g.grid_w - p.wx * g.win_w < g.win_w ? g.grid_w - p.wx * g.win_w : g.win_w;
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
