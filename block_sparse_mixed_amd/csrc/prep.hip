// K1: fused operand preparation.
//
// [DraftAttention2 (arXiv 2609.32628), abstract]: operands for both precision
// phases are prepared in one fused pass; Q and K are pooled (2D average and
// max) for the draft map. [DraftAttention (arXiv 2505.14708), abstract]: Q, K
// and V are reordered so that every 2D window is one contiguous tile.
//
// One workgroup per four consecutive blocks of one (batch*head, tensor), the
// next block's loads in flight while the current one is processed. It reads
// each window's bf16 rows once (8 rows of 16 consecutive raster tokens for an
// 8x16 window), stages them in LDS and writes:
//   - E4M3 codes with one power-of-two scale for the whole block
//     (Q, K slot-major; V channel-major so that PV can contract over slots),
//   - MXFP4 codes with an E8M0 scale per 32 elements along the contraction
//     axis (Q, K along channels; V along slots),
//   - for Q and K, the per-channel mean (fp64, exact sum of bf16 values then
//     one rounding) and maximum over the window's real tokens.
// HBM-bound: ~2 bytes read and ~2 bytes written per element (the codes of
// padded slots included).
#include "common.hpp"

namespace da2 {

struct PrepArgs {
    Geo g;
    const uint16_t* src[3];
    uint8_t* ws;
    Layout L;
};

namespace {

constexpr int kThreads = 256;
constexpr int kPitch = DA2_DPAD + 8;   // bf16 elements per LDS row (272 bytes)
constexpr int kTilesPerGroup = 4;

__device__ __forceinline__ uint32_t abs_bits(uint32_t bf16) { return bf16 & 0x7FFFu; }

}  // namespace

__global__ __launch_bounds__(kThreads) void prep_kernel(PrepArgs a) {
    const Geo& g = a.g;
    const int bh = blockIdx.y;
    const int tz = blockIdx.z;                 // 0 = q, 1 = k, 2 = v
    const int tid = threadIdx.x;
    const int b = bh / g.heads;
    const int h = bh - b * g.heads;

    __shared__ __align__(16) uint16_t tile[DA2_TILE * kPitch];
    __shared__ uint32_t red[kThreads / 64];
    __shared__ double psum[DA2_DPAD];
    __shared__ float pmax[DA2_DPAD];
    __shared__ int sraster[2][DA2_TILE];       // raster index of each slot, -1 for padding (two tiles)

    const uint16_t* src = a.src[tz] + (int64_t)b * g.stride_b + (int64_t)h * g.stride_h;
    // chunk ci = 8 channels of one slot; 16 chunks per slot row
    auto load = [&](uint4 (&chunk)[8], const int* sr) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int ci = tid + kThreads * it;
            const int s = ci >> 4;
            const int cc = ci & 15;
            const int64_t n = sr[s];
            uint4 v = make_uint4(0, 0, 0, 0);
            if (n >= 0 && cc * 8 < g.head_dim) v = *reinterpret_cast<const uint4*>(src + n * g.stride_n + cc * 8);
            chunk[it] = v;
        }
    };
    // A workgroup prepares kTilesPerGroup consecutive blocks; the loads of
    // the next block are issued before the current one is processed, so
    // that one tile's memory latency hides behind the other's work. The
    // window geometry is tabulated once per slot (one integer division
    // each), not per use.
    const int blk0 = blockIdx.x * kTilesPerGroup;
    if (tid < DA2_TILE) sraster[0][tid] = (int)slot_raster(g, block_pos(g, blk0), tid);
    __syncthreads();
    uint4 chunk[8];
    load(chunk, sraster[0]);
#pragma unroll
    for (int t = 0; t < kTilesPerGroup; ++t) {
    const int blk = blk0 + t;
    if (blk >= g.n_blocks) break;
    const BlockPos pos = block_pos(g, blk);
    const int* sr = sraster[t & 1];
    const bool more = t + 1 < kTilesPerGroup && blk + 1 < g.n_blocks;
    if (more && tid < DA2_TILE) sraster[(t + 1) & 1][tid] = (int)slot_raster(g, block_pos(g, blk + 1), tid);

    // ---- stage the tile in LDS ----
    uint32_t amax_bits = 0;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int ci = tid + kThreads * it;
        const int s = ci >> 4;
        const int cc = ci & 15;
        const uint4 v = chunk[it];
        *reinterpret_cast<uint4*>(&tile[s * kPitch + cc * 8]) = v;
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            amax_bits = max(amax_bits, max(abs_bits(w[q] & 0xFFFFu), abs_bits(w[q] >> 16)));
    }
    // ---- block max |x| for the fp8 scale ----
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, off));
    if ((tid & 63) == 0) red[tid >> 6] = amax_bits;
    __syncthreads();
    amax_bits = max(max(red[0], red[1]), max(red[2], red[3]));
    // the next tile's loads go out now, into the registers this tile no
    // longer needs (its raster table is visible after the barrier); this
    // tile is read from LDS from here on
    if (more) load(chunk, sraster[(t + 1) & 1]);
    const int e8 = fp8_exponent(bf16_bits_to_f32(amax_bits));
    const float inv8 = exp2i(-e8);

    const uint64_t tileid = (uint64_t)bh * g.n_blocks + blk;
    if (tid == 0) a.ws[a.L.e8 + (uint64_t)tz * g.bh * g.n_blocks + tileid] = (uint8_t)(e8 + 127);
    if (bh == 0 && tz == 0 && tid < DA2_TILE) {   // geometry only: written once per block
        float* bias = reinterpret_cast<float*>(a.ws + a.L.bias);
        bias[(uint64_t)blk * DA2_TILE + tid] = slot_raster(g, pos, tid) >= 0 ? 0.0f : -__builtin_huge_valf();
        if (blk == 0) bias[(uint64_t)g.n_blocks * DA2_TILE + tid] = -__builtin_huge_valf();   // the empty tile
    }

    if (tz < 2) {
        // ---- row pass (Q, K): E4M3 slot-major and MXFP4 along channels ----
        uint8_t* c8 = a.ws + (tz == 0 ? a.L.q8 : a.L.k8) + tileid * (DA2_TILE * DA2_DPAD);
        uint8_t* c4 = a.ws + (tz == 0 ? a.L.q4 : a.L.k4) + tileid * (DA2_TILE * DA2_DPAD / 2);
        uint8_t* s4 = a.ws + (tz == 0 ? a.L.sq4 : a.L.sk4) + tileid * (DA2_TILE * DA2_DPAD / 32);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int ci = tid + kThreads * it;
            const int s = ci >> 4;
            const int cc = ci & 15;
            const uint4 v = *reinterpret_cast<const uint4*>(&tile[s * kPitch + cc * 8]);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            float x[8];
            uint32_t gmax = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[2 * q] = bf16_bits_to_f32(w[q] & 0xFFFFu);
                x[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
                gmax = max(gmax, max(abs_bits(w[q] & 0xFFFFu), abs_bits(w[q] >> 16)));
            }
            uint2 o8;
            o8.x = pack_fp8x4(x[0] * inv8, x[1] * inv8, x[2] * inv8, x[3] * inv8);
            o8.y = pack_fp8x4(x[4] * inv8, x[5] * inv8, x[6] * inv8, x[7] * inv8);
            *reinterpret_cast<uint2*>(c8 + s * DA2_DPAD + cc * 8) = o8;
            // 32-channel group = 4 consecutive lanes
            gmax = max(gmax, (uint32_t)__shfl_xor((int)gmax, 1));
            gmax = max(gmax, (uint32_t)__shfl_xor((int)gmax, 2));
            const int e4 = fp4_exponent(bf16_bits_to_f32(gmax));
            const float inv4 = exp2i(-e4);
            float y[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) y[q] = x[q] * inv4;
            *reinterpret_cast<uint32_t*>(c4 + s * (DA2_DPAD / 2) + cc * 4) = pack_fp4x8(y);
            if ((cc & 3) == 0) s4[s * (DA2_DPAD / 32) + (cc >> 2)] = (uint8_t)(e4 + 127);
        }
    }
    __syncthreads();

    // ---- column pass: thread = (channel, half of the slots) ----
    const int c = tid & (DA2_DPAD - 1);
    const int half = tid >> 7;
    if (tz == 2) {
        uint8_t* c8 = a.ws + a.L.v8t + tileid * (DA2_DPAD * DA2_TILE) + c * DA2_TILE + half * 64;
        uint8_t* c4 = a.ws + a.L.v4t + tileid * (DA2_DPAD * DA2_TILE / 2) + c * (DA2_TILE / 2) + half * 32;
        uint8_t* s4 = a.ws + a.L.sv4t + tileid * (DA2_DPAD * DA2_TILE / 32) + c * (DA2_TILE / 32) + half * 2;
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
            float x[32];
            uint32_t gmax = 0;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const uint32_t bits = tile[(half * 64 + grp * 32 + j) * kPitch + c];
                x[j] = bf16_bits_to_f32(bits);
                gmax = max(gmax, abs_bits(bits));
            }
            uint4 o8a, o8b;
            o8a.x = pack_fp8x4(x[0] * inv8, x[1] * inv8, x[2] * inv8, x[3] * inv8);
            o8a.y = pack_fp8x4(x[4] * inv8, x[5] * inv8, x[6] * inv8, x[7] * inv8);
            o8a.z = pack_fp8x4(x[8] * inv8, x[9] * inv8, x[10] * inv8, x[11] * inv8);
            o8a.w = pack_fp8x4(x[12] * inv8, x[13] * inv8, x[14] * inv8, x[15] * inv8);
            o8b.x = pack_fp8x4(x[16] * inv8, x[17] * inv8, x[18] * inv8, x[19] * inv8);
            o8b.y = pack_fp8x4(x[20] * inv8, x[21] * inv8, x[22] * inv8, x[23] * inv8);
            o8b.z = pack_fp8x4(x[24] * inv8, x[25] * inv8, x[26] * inv8, x[27] * inv8);
            o8b.w = pack_fp8x4(x[28] * inv8, x[29] * inv8, x[30] * inv8, x[31] * inv8);
            *reinterpret_cast<uint4*>(c8 + grp * 32) = o8a;
            *reinterpret_cast<uint4*>(c8 + grp * 32 + 16) = o8b;
            const int e4 = fp4_exponent(bf16_bits_to_f32(gmax));
            const float inv4 = exp2i(-e4);
            float y[32];
#pragma unroll
            for (int j = 0; j < 32; ++j) y[j] = x[j] * inv4;
            uint4 o4;
            o4.x = pack_fp4x8(y);
            o4.y = pack_fp4x8(y + 8);
            o4.z = pack_fp4x8(y + 16);
            o4.w = pack_fp4x8(y + 24);
            *reinterpret_cast<uint4*>(c4 + grp * 16) = o4;
            s4[grp] = (uint8_t)(e4 + 127);
        }
    } else {
        // pooling over the real tokens: fp64 sums of bf16 values, signed max.
        // A bf16 value has 8 significant bits, so the sums are exact (and the
        // four partial sums' order irrelevant) while a channel's values lie
        // within 2^38 of each other. Padded slots hold zeros in the tile,
        // which leave the sums unchanged; the max skips them.
        double sum4[4] = {0.0, 0.0, 0.0, 0.0};
        float mx4[4] = {-__builtin_huge_valf(), -__builtin_huge_valf(), -__builtin_huge_valf(),
                        -__builtin_huge_valf()};
#pragma unroll 4
        for (int s = half * 64; s < half * 64 + 64; ++s) {
            const float x = bf16_bits_to_f32(tile[s * kPitch + c]);
            sum4[s & 3] += (double)x;
            mx4[s & 3] = sr[s] >= 0 ? fmaxf(mx4[s & 3], x) : mx4[s & 3];
        }
        double sum = (sum4[0] + sum4[1]) + (sum4[2] + sum4[3]);
        float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
        if (half == 1) {
            psum[c] = sum;
            pmax[c] = mx;
        }
        __syncthreads();
        if (half == 0) {
            sum += psum[c];
            mx = fmaxf(mx, pmax[c]);
            const bool real = c < g.head_dim;
            const double mean = real ? sum / (double)block_count(g, pos) : 0.0;
            const double maxv = real ? (double)mx : 0.0;
            double* pool = reinterpret_cast<double*>(a.ws + a.L.pool);
            const uint64_t plane = (uint64_t)g.bh * g.n_blocks * DA2_DPAD;
            pool[(2 * tz) * plane + tileid * DA2_DPAD + c] = mean;
            pool[(2 * tz + 1) * plane + tileid * DA2_DPAD + c] = maxv;
        }
    }
    // the tile, the reduction slots and this tile's raster table are reused
    __syncthreads();
    }
}

hipError_t launch_prep(const Geo& g, const Layout& L, const void* q, const void* k, const void* v,
                       void* ws, hipStream_t stream) {
    PrepArgs a;
    a.g = g;
    a.src[0] = static_cast<const uint16_t*>(q);
    a.src[1] = static_cast<const uint16_t*>(k);
    a.src[2] = static_cast<const uint16_t*>(v);
    a.ws = static_cast<uint8_t*>(ws);
    a.L = L;
    return launch_kernel(prep_kernel, dim3((g.n_blocks + kTilesPerGroup - 1) / kTilesPerGroup, g.bh, 3), dim3(kThreads), 0,
                         stream, a);
}

}  // namespace da2
