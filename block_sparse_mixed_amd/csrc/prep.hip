// K1: fused operand preparation.
//
// [DraftAttention2 (arXiv 2609.32628), abstract]: operands for both precision
// phases are prepared in one fused pass; Q and K are pooled (2D average and
// max) for the draft map. [DraftAttention (arXiv 2505.14708), abstract]: Q, K
// and V are reordered so that every 2D window is one contiguous tile.
//
// One round of resident workgroups, each preparing a run of consecutive
// blocks, the next block's loads in flight while the current one is
// processed. It reads
// each window's bf16 rows once (8 rows of 16 consecutive raster tokens for an
// 8x16 window) and writes:
//   - E4M3 codes with one power-of-two scale for the whole block
//     (Q, K slot-major; V channel-major so that PV can contract over slots),
//   - MXFP4 codes with an E8M0 scale per 32 elements along the contraction
//     axis (Q, K along channels; V along slots),
//   - for Q and K, the per-channel mean (fp64, exact sum of bf16 values then
//     one rounding) and maximum over the window's real tokens.
// HBM-bound: ~2 bytes read and ~2 bytes written per element (the codes of
// padded slots included). The instruction count per element is what keeps it
// from that bound, so the conversions run straight from the packed bf16 words
// (one instruction per two values, the scale applied by the conversion),
// magnitudes are compared two at a time as 16-bit integers, and Q and K never
// pass through LDS: a thread's eight channels of eight slots stay in its
// registers from the load to the stores, and the pooling over slots ends in
// lane reductions.
#include <atomic>

#include "common.hpp"

namespace da2 {

struct PrepArgs {
    Geo g;
    const uint16_t* src[3];
    uint8_t* ws;
    Layout L;
};

namespace {

typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef short v2s16 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr uint32_t kAbs2 = 0x7FFF7FFFu;   // magnitude bits of two packed bf16 values
// Scale exponents from here up convert with the conversion's own scale
// operand: 2^e is a normal float, and a bf16 subnormal divided by it stays
// below 2^-26, far under the smallest nonzero code, whether or not the
// hardware flushes it. Smaller exponents (blocks or groups of magnitude below
// about 2^-92) multiply by 2^-e in fp32 first.
constexpr int kMinScaledExp = -100;

// Streaming accesses (the nt bit) for the V kernel: its bf16 input is read
// once, and its codes are read by the attention kernel only after some
// hundreds of MB have passed through the caches, so neither gains from
// staying in L2. Measured in the step (interleaved medians of the
// preparation): 0.2006 ms with plain accesses, 0.1996 with streaming loads
// and code stores in both kernels, 0.1967 with them in the V kernel only
// (the Q/K kernel then ran slower after an attention launch).
__device__ __forceinline__ uint4 load_stream(const void* p) {
    const v4u32 t = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void store_stream(void* p, uint4 v) {
    __builtin_nontemporal_store((v4u32){v.x, v.y, v.z, v.w}, reinterpret_cast<v4u32*>(p));
}
__device__ __forceinline__ void store_stream(void* p, uint2 v) {
    __builtin_nontemporal_store((v2u32){v.x, v.y}, reinterpret_cast<v2u32*>(p));
}

// Per-half unsigned maximum of two pairs of 16-bit values (V_PK_MAX_U16).
__device__ __forceinline__ uint32_t max2_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_max(__builtin_bit_cast(v2u16, a), __builtin_bit_cast(v2u16, b)));
}
__device__ __forceinline__ uint32_t max_half(uint32_t a) { return max(a & 0xFFFFu, a >> 16); }
// IEEE maximum (V_MAXIMUM_F32): the inputs are never NaN, so it is the usual
// max, without the quieting instructions fmaxf adds in front of each input.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Eight bf16 values (low half of each word first) -> eight E4M3 codes of
// x / scale. V_CVT_SCALEF32_PK_FP8_BF16 divides by its scale operand and
// rounds to nearest even; for scale = 2^e the quotient is exact, so the codes
// are RNE(x * 2^-e). The first conversion of a word pair writes the low 16
// bits of its "old" operand and the second the high 16 bits: any old value
// will do.
__device__ __forceinline__ uint2 fp8x8_scaled(uint4 v, float scale) {
    v2s16 a = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(v2s16, v.x),
                                                        __builtin_bit_cast(v2bf16, v.x), scale, false);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(a, __builtin_bit_cast(v2bf16, v.y), scale, true);
    v2s16 b = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(v2s16, v.z),
                                                        __builtin_bit_cast(v2bf16, v.z), scale, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(b, __builtin_bit_cast(v2bf16, v.w), scale, true);
    return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

// Eight bf16 values -> eight E2M1 codes of x / scale (round to nearest even,
// saturating at 6), low nibble first; byte i from word i.
__device__ __forceinline__ uint32_t fp4x8_scaled(uint4 v, float scale) {
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(v.x, __builtin_bit_cast(v2bf16, v.x), scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(v2bf16, v.y), scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(v2bf16, v.z), scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(v2bf16, v.w), scale, 3);
    return w;
}

// The same codes for scale exponents below kMinScaledExp: the values times
// 2^-e in fp32 (exact: bf16 values have 8 significant bits), then converted.
__device__ __forceinline__ void unpack8(uint4 v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        x[2 * q] = __uint_as_float(w[q] << 16);
        x[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ uint2 fp8x8_small(uint4 v, int e) {
    const float inv = exp2i(-e);
    float x[8];
    unpack8(v, x);
    return make_uint2(pack_fp8x4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv),
                      pack_fp8x4(x[4] * inv, x[5] * inv, x[6] * inv, x[7] * inv));
}
__device__ __forceinline__ uint32_t fp4x8_small(uint4 v, int e) {
    const float inv = exp2i(-e);
    float x[8];
    unpack8(v, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] *= inv;
    return pack_fp4x8(x);
}

// Sums and maxima over the lane pairs (l, l ^ 16) and (l, l ^ 32) through
// the permlane swaps: a swap of two copies of a value gives every lane both
// values of its pair, so both lanes compute the same result in the same order.
__device__ __forceinline__ double add_swap16(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    return __builtin_bit_cast(double, ((uint64_t)hi[0] << 32) | lo[0]) +
           __builtin_bit_cast(double, ((uint64_t)hi[1] << 32) | lo[1]);
}
__device__ __forceinline__ double add_swap32(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    return __builtin_bit_cast(double, ((uint64_t)hi[0] << 32) | lo[0]) +
           __builtin_bit_cast(double, ((uint64_t)hi[1] << 32) | lo[1]);
}
__device__ __forceinline__ float max_swap16(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float max_swap32(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
}

// Chunk swizzle of the staged V tile: chunk cc of slot s sits at chunk
// cc ^ vswz(s). The column pass's 16 lanes per read take slots from eight
// groups of 16 and two neighbouring chunks; the swizzle spreads them over all
// sixteen chunk positions.
__device__ __forceinline__ int vswz(int s) { return ((s >> 4) & 7) << 1; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
    return v;
}

}  // namespace

// Tile i of a kernel: tensor, batch*head and block, in (tensor, b*h, block)
// order.
struct TileRef {
    int tz, bh, blk;
};

// kV false: Q and K; kV true: V. Two kernels, so that each gets the
// registers of its own path. Workgroup w prepares the kernel's tiles
// [w * per, (w + 1) * per), with per chosen on the host so that the grid is
// one round of resident workgroups (no partly filled last round).
template <bool kV>
__global__ __launch_bounds__(kThreads, 4) void prep_kernel(PrepArgs a, int per) {
    const Geo& g = a.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int plane = g.bh * g.n_blocks;       // tiles per tensor
    const int total = kV ? plane : 2 * plane;
    const int first = blockIdx.x * per;
    const int last = min(first + per, total);
    if (first >= total) return;
    auto decode = [&](int i) __attribute__((always_inline)) {
        TileRef r;
        r.tz = kV ? 2 : (i >= plane ? 1 : 0);
        const int rem = (kV || i < plane) ? i : i - plane;
        r.bh = rem / g.n_blocks;
        r.blk = rem - r.bh * g.n_blocks;
        return r;
    };
    auto src_of = [&](const TileRef& r) __attribute__((always_inline)) {
        const int b = r.bh / g.heads;
        const int h = r.bh - b * g.heads;
        return a.src[r.tz] + (int64_t)b * g.stride_b + (int64_t)h * g.stride_h;
    };

    // V tiles are staged here for the transposition; Q and K use the space
    // for the four waves' pooling partials.
    __shared__ __align__(16) uint8_t smem[kV ? DA2_TILE * DA2_DPAD * 2 : 4 * DA2_DPAD * (8 + 4)];
    __shared__ uint32_t red[kThreads / 64];
    __shared__ int sraster[2][DA2_TILE];       // raster index of each slot, -1 for padding (two tiles)
    double* psum = reinterpret_cast<double*>(smem);                     // [4 waves][128 channels]
    float* pmax = reinterpret_cast<float*>(smem + 4 * DA2_DPAD * 8);    // [4 waves][128 channels]

    // Chunk it of a thread: channels 8 cc .. 8 cc + 7 (cc = tid % 16) of
    // slot tid / 16 + 16 it. Bit it of the real mask: the slot holds a token.
    const int cc = tid & 15;
    const bool chan_real = cc * 8 < g.head_dim;
    auto load_one = [&](uint4& c, uint32_t& realm, const uint16_t* src, const int* sr, int it)
                        __attribute__((always_inline)) {
        const int s = (tid >> 4) + 16 * it;
        const int64_t n = sr[s];
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n >= 0 && chan_real) v = kV ? load_stream(src + n * g.stride_n + cc * 8)
                                        : *reinterpret_cast<const uint4*>(src + n * g.stride_n + cc * 8);
        realm |= (n >= 0 ? 1u : 0u) << it;
        c = v;
    };
    // The next tile's loads are in flight while the current one is
    // processed, so that one tile's memory latency hides behind the other's
    // work. For V they go out once the tile is staged in LDS; for Q and K
    // chunk by chunk, each into the registers of the chunk just finished, so
    // that the two tiles together hold eight chunks' registers. The window
    // geometry is tabulated once per slot (one integer division each), not
    // per use.
    TileRef nx = decode(first);
    if (tid < DA2_TILE) sraster[0][tid] = (int)slot_raster(g, block_pos(g, nx.blk), tid);
    __syncthreads();
    uint4 chunk[8];
    uint32_t realm = 0;
    {
        const uint16_t* src = src_of(nx);
#pragma unroll
        for (int it = 0; it < 8; ++it) load_one(chunk[it], realm, src, sraster[0], it);
    }
    for (int i = first, k = 0; i < last; ++i, ++k) {
    const TileRef tr = nx;
    const int tz = tr.tz, bh = tr.bh, blk = tr.blk;
    const BlockPos pos = block_pos(g, blk);
    const bool more = i + 1 < last;
    if (more) nx = decode(i + 1);
    if (more && tid < DA2_TILE) sraster[(k + 1) & 1][tid] = (int)slot_raster(g, block_pos(g, nx.blk), tid);
    const uint16_t* src_next = src_of(nx);
    const uint64_t tileid = (uint64_t)bh * g.n_blocks + blk;

    // ---- magnitudes: per chunk (two per word), and the block's ----
    uint32_t cmax[8];
    uint32_t amax2 = 0;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const uint4 v = chunk[it];
        cmax[it] = max2_u16(max2_u16(v.x & kAbs2, v.y & kAbs2), max2_u16(v.z & kAbs2, v.w & kAbs2));
        amax2 = max2_u16(amax2, cmax[it]);
    }
    if constexpr (kV) {
        // V: stage the tile for the column pass, rows of 256 bytes, chunk
        // cc of slot s at chunk cc ^ vswz(s)
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int s = (tid >> 4) + 16 * it;
            *reinterpret_cast<uint4*>(smem + s * 256 + ((cc ^ vswz(s)) << 4)) = chunk[it];
        }
    }
    {
        const uint32_t m = wave_max_u32(max_half(amax2));
        if (lane == 0) red[wv] = m;
    }
    __syncthreads();
    const uint32_t amax_bits =
        (uint32_t)__builtin_amdgcn_readfirstlane((int)max(max(red[0], red[1]), max(red[2], red[3])));
    // (the next tile's raster table is visible after the barrier)
    const int* sr_next = sraster[(k + 1) & 1];
    const uint32_t realm_cur = realm;
    realm = 0;
    const int e8 = fp8_exponent(bf16_bits_to_f32(amax_bits));
    const bool small8 = e8 < kMinScaledExp && amax_bits != 0;

    if (tid == 0) a.ws[a.L.e8 + (uint64_t)tz * g.bh * g.n_blocks + tileid] = (uint8_t)(e8 + 127);
    if (bh == 0 && tz == 0 && tid < DA2_TILE) {   // geometry only: written once per block
        float* bias = reinterpret_cast<float*>(a.ws + a.L.bias);
        bias[(uint64_t)blk * DA2_TILE + tid] = slot_raster(g, pos, tid) >= 0 ? 0.0f : -__builtin_huge_valf();
        if (blk == 0) bias[(uint64_t)g.n_blocks * DA2_TILE + tid] = -__builtin_huge_valf();   // the empty tile
    }

    if constexpr (!kV) {
        // ---- Q, K: E4M3 slot-major, MXFP4 along channels, pooling ----
        uint8_t* c8 = a.ws + (tz == 0 ? a.L.q8 : a.L.k8) + tileid * (DA2_TILE * DA2_DPAD);
        uint8_t* c4 = a.ws + (tz == 0 ? a.L.q4 : a.L.k4) + tileid * (DA2_TILE * DA2_DPAD / 2);
        uint8_t* s4 = a.ws + (tz == 0 ? a.L.sq4 : a.L.sk4) + tileid * (DA2_TILE * DA2_DPAD / 32);
        const uint32_t o8 = (uint32_t)(tid >> 4) * DA2_DPAD + cc * 8;
        const uint32_t o4 = (uint32_t)(tid >> 4) * (DA2_DPAD / 2) + cc * 4;
        const uint32_t os4 = (uint32_t)(tid >> 4) * (DA2_DPAD / 32) + (cc >> 2);
        // pooling over the real tokens: fp64 sums of bf16 values, signed max.
        // A bf16 value has 8 significant bits, so the sums are exact (and
        // their order irrelevant) while a channel's values lie within 2^38
        // of each other. Padded slots hold zeros, which leave the sums
        // unchanged; the max skips them.
        double sum[8];
        float mx[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            sum[j] = 0.0;
            mx[j] = -__builtin_huge_valf();
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            // slot tid / 16 + 16 it: the part 16 it of the address is
            // uniform and joins the scalar base, so that one 32-bit lane
            // offset per array serves every chunk
            const uint4 v = chunk[it];
            uint2 w8;
            if (small8)
                w8 = fp8x8_small(v, e8);
            else
                w8 = fp8x8_scaled(v, exp2i(max(e8, kMinScaledExp)));
            *reinterpret_cast<uint2*>(c8 + 16 * DA2_DPAD * it + o8) = w8;
            // 32-channel group = 4 consecutive lanes (DPP quad permutations)
            uint32_t gm = cmax[it];
            gm = max2_u16(gm, (uint32_t)__builtin_amdgcn_mov_dpp((int)gm, 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
            gm = max2_u16(gm, (uint32_t)__builtin_amdgcn_mov_dpp((int)gm, 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
            gm = max_half(gm);
            const int e4 = fp4_exponent(bf16_bits_to_f32(gm));
            uint32_t w4;
            if (e4 < kMinScaledExp && gm != 0)
                w4 = fp4x8_small(v, e4);
            else
                w4 = fp4x8_scaled(v, exp2i(max(e4, kMinScaledExp)));
            *reinterpret_cast<uint32_t*>(c4 + 16 * (DA2_DPAD / 2) * it + o4) = w4;
            if ((cc & 3) == 0) s4[16 * (DA2_DPAD / 32) * it + os4] = (uint8_t)(e4 + 127);
            float x[8];
            unpack8(v, x);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                sum[j] += (double)x[j];
                asm volatile("" : "+v"(sum[j]));   // summed here, not sunk past the loop with x live
            }
            if ((realm_cur >> it) & 1u) {
#pragma unroll
                for (int j = 0; j < 8; ++j) mx[j] = vmax(mx[j], x[j]);
            }
            // the next tile's chunk into this chunk's registers, now free
            if (more) load_one(chunk[it], realm, src_next, sr_next, it);
            __builtin_amdgcn_sched_barrier(0);   // one chunk at a time: bounds the live registers
        }
        // lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same channels: reduce, then
        // the four waves' partials through LDS (free since the last tile's
        // closing barrier)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            sum[j] = add_swap32(add_swap16(sum[j]));
            mx[j] = max_swap32(max_swap16(mx[j]));
            __builtin_amdgcn_sched_barrier(0);   // one channel at a time
        }
        if (lane < 16) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                psum[wv * DA2_DPAD + cc * 8 + j] = sum[j];
                pmax[wv * DA2_DPAD + cc * 8 + j] = mx[j];
            }
        }
        __syncthreads();
        if (tid < DA2_DPAD) {
            const int c = tid;
            const double s = (psum[c] + psum[DA2_DPAD + c]) + (psum[2 * DA2_DPAD + c] + psum[3 * DA2_DPAD + c]);
            const float m = vmax(vmax(pmax[c], pmax[DA2_DPAD + c]), vmax(pmax[2 * DA2_DPAD + c], pmax[3 * DA2_DPAD + c]));
            const bool real = c < g.head_dim;
            double* pool = reinterpret_cast<double*>(a.ws + a.L.pool);
            const uint64_t plane = (uint64_t)g.bh * g.n_blocks * DA2_DPAD;
            pool[(2 * tz) * plane + tileid * DA2_DPAD + c] = real ? s / (double)block_count(g, pos) : 0.0;
            pool[(2 * tz + 1) * plane + tileid * DA2_DPAD + c] = real ? (double)m : 0.0;
        }
    } else {
        // ---- V: E4M3 channel-major, MXFP4 along slots ----
        // Two passes of 16 channels per wave. Lane: channels c0, c0 + 1
        // (c0 = 32 wv + 16 pass + 2 (lane / 8)) over the 16 slots 16 sg ..
        // 16 sg + 15 (sg = lane % 8; lanes sg and sg ^ 1 share an MXFP4
        // group). A store then writes 16 (E4M3) or 8 (E2M1) bytes at column
        // 16 sg (8 sg) of a channel row: eight lanes fill one row. The
        // swizzle puts the 16 lanes of a read on 16 different 16-byte bank
        // groups.
        if (more) {
#pragma unroll
            for (int it = 0; it < 8; ++it) load_one(chunk[it], realm, src_next, sr_next, it);
        }
        const int sg = lane & 7;
        const float sc8 = exp2i(max(e8, kMinScaledExp));
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int c0 = 32 * wv + 16 * pass + 2 * (lane >> 3);
            const int rd = 16 * sg * 256 + (((c0 >> 3) ^ vswz(16 * sg)) << 4) + (c0 & 7) * 2;
            uint32_t wrd[16];   // slot 16 sg + j: channel c0 in the low half, c0 + 1 in the high
#pragma unroll
            for (int j = 0; j < 16; ++j) wrd[j] = *reinterpret_cast<const uint32_t*>(smem + rd + j * 256);
            uint32_t am = 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) am = max2_u16(am, wrd[j] & kAbs2);
            am = max2_u16(am, (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {
                const int c = c0 + ch;
                // slot pairs (2 i, 2 i + 1) of channel c as packed bf16 words:
                // V_PERM_B32 takes bytes 0-1 (or 2-3) of the even slot's word,
                // then of the odd's
                const uint32_t sel = ch ? 0x07060302u : 0x05040100u;
                uint4 pr[2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    pr[i] = make_uint4(__builtin_amdgcn_perm(wrd[8 * i + 1], wrd[8 * i], sel),
                                       __builtin_amdgcn_perm(wrd[8 * i + 3], wrd[8 * i + 2], sel),
                                       __builtin_amdgcn_perm(wrd[8 * i + 5], wrd[8 * i + 4], sel),
                                       __builtin_amdgcn_perm(wrd[8 * i + 7], wrd[8 * i + 6], sel));
                // uniform bases, 32-bit lane offsets
                uint8_t* c8 = a.ws + a.L.v8t + tileid * (DA2_DPAD * DA2_TILE) + (uint32_t)(c * DA2_TILE + 16 * sg);
                uint8_t* c4 = a.ws + a.L.v4t + tileid * (DA2_DPAD * DA2_TILE / 2) + (uint32_t)(c * (DA2_TILE / 2) + 8 * sg);
                uint8_t* s4 = a.ws + a.L.sv4t + tileid * (DA2_DPAD * DA2_TILE / 32) + (uint32_t)(c * (DA2_TILE / 32) + (sg >> 1));
                // the rare small-scale paths read the tile again, four or
                // eight values at a time, so that they hold few registers
                auto col = [&](int j) __attribute__((always_inline)) {
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(smem + rd + j * 256);
                    return __uint_as_float(ch ? (w & 0xFFFF0000u) : (w << 16));
                };
                if (small8) {
                    const float inv = exp2i(-e8);
#pragma unroll 1
                    for (int j = 0; j < 16; j += 4)
                        *reinterpret_cast<uint32_t*>(c8 + j) =
                            pack_fp8x4(col(j) * inv, col(j + 1) * inv, col(j + 2) * inv, col(j + 3) * inv);
                } else {
                    const uint2 lo = fp8x8_scaled(pr[0], sc8), hi = fp8x8_scaled(pr[1], sc8);
                    store_stream(c8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                }
                const uint32_t gm = ch ? am >> 16 : am & 0xFFFFu;
                const int e4 = fp4_exponent(bf16_bits_to_f32(gm));
                if (e4 < kMinScaledExp && gm != 0) {
                    const float inv = exp2i(-e4);
#pragma unroll 1
                    for (int j = 0; j < 16; j += 8) {
                        float y[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) y[e] = col(j + e) * inv;
                        *reinterpret_cast<uint32_t*>(c4 + j / 2) = pack_fp4x8(y);
                    }
                } else {
                    const float sc = exp2i(max(e4, kMinScaledExp));
                    store_stream(c4, make_uint2(fp4x8_scaled(pr[0], sc), fp4x8_scaled(pr[1], sc)));
                }
                if ((sg & 1) == 0) *s4 = (uint8_t)(e4 + 127);
                __builtin_amdgcn_sched_barrier(0);   // one channel at a time
            }
        }
    }
    // the tile, the pooling partials, the reduction slots and this tile's
    // raster table are reused
    __syncthreads();
    }
}

namespace {

// Workgroups of a prep kernel resident on the device of the stream at once
// (occupancy times compute units), looked up once per device.
template <bool kV>
int resident_groups(hipStream_t stream) {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess && hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev >= 0 && dev < 64)
        if (const int c = cache[dev].load(std::memory_order_relaxed); c > 0) return c;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prep_kernel<kV>, kThreads, 0) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    const int n = cus * per_cu;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

template <bool kV>
hipError_t launch_one(const PrepArgs& a, hipStream_t stream) {
    const int total = (kV ? 1 : 2) * a.g.bh * a.g.n_blocks;
    const int slots = resident_groups<kV>(stream);
    const int per = (total + slots - 1) / slots;
    const int groups = (total + per - 1) / per;
    return launch_kernel(prep_kernel<kV>, dim3(groups), dim3(kThreads), 0, stream, a, per);
}

}  // namespace

hipError_t launch_prep(const Geo& g, const Layout& L, const void* q, const void* k, const void* v,
                       void* ws, hipStream_t stream) {
    PrepArgs a;
    a.g = g;
    a.src[0] = static_cast<const uint16_t*>(q);
    a.src[1] = static_cast<const uint16_t*>(k);
    a.src[2] = static_cast<const uint16_t*>(v);
    a.ws = static_cast<uint8_t*>(ws);
    a.L = L;
    if (hipError_t e = launch_one<false>(a, stream); e != hipSuccess) return e;
    return launch_one<true>(a, stream);
}

}  // namespace da2
