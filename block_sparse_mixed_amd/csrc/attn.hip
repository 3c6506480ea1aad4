// K3: block-sparse flash attention with an fp8 phase and an MXFP4 phase.
//
// [DraftAttention2 (arXiv 2609.32628), abstract]: one attention kernel with
// precision-specific phases that share data movement, the softmax statistics
// and the output accumulator; 8-bit compute on the top-ranked blocks, 4-bit on
// the other retained blocks, nothing on skipped blocks. [DraftAttention
// (arXiv 2505.14708), abstract]: outputs return to the original token order.
//
// Work decomposition (gfx950, wave64):
//   one workgroup = one query block (128 slots) of one (batch, head); 4 waves,
//   wave w owns query slots 32w .. 32w+31 as two 16-query tiles u.
//   Per key tile (128 slots) the workgroup stages K and V^T in LDS once and
//   every wave runs
//     S^T = K . Q^T        fp8 phase: 32 x V_MFMA_F32_16X16X32_BF16 per query
//                          tile on the E4M3 values decoded to bf16 (exact);
//                          MXFP4 phase: 8 x V_MFMA_SCALE_F32_16X16X128_F8F6F4
//     softmax (base 2, integer running max, lane-local rescale)
//     O^T += V^T . P^T     8 scaled f8f6f4 MFMAs (E4M3 or E2M1 operands), plus
//                          one with an all-ones A that yields the row sum
//                          l = sum P~ in the same lanes as O.
//   The fp8 phase's QK^T runs on bf16 MFMAs because the f8f6f4 MFMA keeps only
//   about 12 bits below its largest product when it sums fp8 products: with
//   outlier channels the scores move by ~1e-2 (log2 units), enough to flip the
//   rounding of many P codes. Its PV product stays fp8: nothing is decided
//   from its rounding.
//   Computing S transposed makes each lane hold 32 keys of one query, which
//   is exactly the B-operand layout of the PV product: P never leaves the
//   lane, the MXFP4 group of P is the lane's own 32 values, and the max
//   reduction needs two cross-lane steps (xor 16, xor 32).
//
// Operand layouts (measured on gfx950): a 16x16x128 fp8 operand lane l holds
// row l%16 and bytes j -> k = 64*(j/16) + 16*(l/16) + j%16; an fp4 operand
// lane l holds row l%16 and nibble j -> k = 32*(l/16) + j; the E8M0 scale of
// lane l belongs to (row l%16, k-block l/16); D lane l element e is
// D[4*(l/16) + e][l%16]. The key slot fed to A-row r of key tile t is chosen
// so that P's register order matches the PV k order:
//   fp8:  slot = 64*(t/4) + 16*(r/4) + 4*(t%4) + r%4
//   fp4:  slot = 32*(r/4) + 4*t + r%4          (k-block g = slots 32g..32g+31)
#include "common.hpp"

namespace da2 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

struct AttnArgs {
    Geo g;
    const uint8_t* ws;
    Layout L;
    void* out;
    int out_fp32;
};

namespace {

constexpr int kThreads = 256;
constexpr int kFmtFp8 = 0;
constexpr int kFmtFp4 = 4;
constexpr float kLog2E = 1.4426950408889634f;
constexpr float kLog2Six = 2.5849625007211562f;

// LDS swizzles (16-byte chunk index XOR a row function) so that the eight
// lanes served together by a 128-bit LDS read hit distinct banks.
__device__ __forceinline__ int swz_k8(int s) { return (s & 3) | ((s >> 2) & 4); }
__device__ __forceinline__ int swz_v8(int c) { return c & 7; }
__device__ __forceinline__ int swz_k4(int s) { return ((s >> 1) & 1) | ((s >> 4) & 2); }
__device__ __forceinline__ int swz_v4(int c) { return (c >> 1) & 3; }

__device__ __forceinline__ int slot_fp8(int t, int r) { return 64 * (t >> 2) + 16 * (r >> 2) + 4 * (t & 3) + (r & 3); }
__device__ __forceinline__ int slot_fp4(int t, int r) { return 32 * (r >> 2) + 4 * t + (r & 3); }

__device__ __forceinline__ v8i load_lds_pair(const uint8_t* lds, int off_a, int off_b) {
    const uint4 x = *reinterpret_cast<const uint4*>(lds + off_a);
    const uint4 y = *reinterpret_cast<const uint4*>(lds + off_b);
    v8i r;
    r[0] = (int)x.x; r[1] = (int)x.y; r[2] = (int)x.z; r[3] = (int)x.w;
    r[4] = (int)y.x; r[5] = (int)y.y; r[6] = (int)y.z; r[7] = (int)y.w;
    return r;
}

__device__ __forceinline__ v8i load_lds_one(const uint8_t* lds, int off) {
    const uint4 x = *reinterpret_cast<const uint4*>(lds + off);
    v8i r;
    r[0] = (int)x.x; r[1] = (int)x.y; r[2] = (int)x.z; r[3] = (int)x.w;
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
    return r;
}

__device__ __forceinline__ float wave_max_4groups(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// Whether every slot of block blk holds a real token.
__device__ __forceinline__ bool block_full(const Geo& g, int blk) {
    return g.block_size == DA2_TILE && block_count(g, block_pos(g, blk)) == DA2_TILE;
}

__device__ __forceinline__ bool slot_real(const Geo& g, const BlockPos& p, int s) {
    if (s >= g.block_size) return false;
    const int iy = s / g.win_w;
    const int ix = s - iy * g.win_w;
    return p.wy * g.win_h + iy < g.grid_h && p.wx * g.win_w + ix < g.grid_w;
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

}  // namespace

__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
    const Geo& g = a.g;
    const int qb = blockIdx.x;
    const int bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int r = lane & 15;
    const int g4 = lane >> 4;
    const int nb = g.n_blocks;

    __shared__ __align__(16) uint8_t kt[DA2_TILE * DA2_DPAD * 2];   // bf16 K (fp8 phase) or E2M1 K
    __shared__ __align__(16) uint8_t vt[DA2_DPAD * DA2_TILE];
    __shared__ uint8_t ks4[DA2_TILE * 4];
    __shared__ uint8_t vs4[DA2_DPAD * 4];

    const uint8_t* ws = a.ws;
    const uint64_t qtile = (uint64_t)bh * nb + qb;
    const uint8_t* e8 = ws + a.L.e8;
    const uint64_t eplane = (uint64_t)g.bh * nb;
    const int e_q8 = (int)e8[qtile] - 127;

    // Q operands (B of S^T = K Q^T): query slot 32w + 16u + r
    // bf16 operand of a 16x16x32 MFMA: lane (r, g4) takes channels 32kk + 8g4 .. +8
    // of its row for k-step kk, the same assignment for A and B.
    v8bf qbop[2][4];
    v8i q4op[2];
    int q4sc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int qs = 32 * w + 16 * u + r;
        const uint8_t* rowb = ws + a.L.qb + (qtile * (DA2_TILE * DA2_DPAD) + qs * DA2_DPAD) * 2;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qbop[u][kk] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(rowb + 64 * kk + 16 * g4));
        const uint8_t* row4 = ws + a.L.q4 + qtile * (DA2_TILE * DA2_DPAD / 2) + qs * (DA2_DPAD / 2);
        const uint4 x4 = *reinterpret_cast<const uint4*>(row4 + 16 * g4);
        q4op[u][0] = (int)x4.x; q4op[u][1] = (int)x4.y; q4op[u][2] = (int)x4.z; q4op[u][3] = (int)x4.w;
        q4op[u][4] = 0; q4op[u][5] = 0; q4op[u][6] = 0; q4op[u][7] = 0;
        q4sc[u] = (int)ws[a.L.sq4 + qtile * (DA2_TILE * DA2_DPAD / 32) + qs * (DA2_DPAD / 32) + g4];
    }

    float m[2] = {-__builtin_huge_valf(), -__builtin_huge_valf()};
    v4f acc[2][8];
    v4f lsum[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        lsum[u] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[u][ct] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
    const float c_lo = (float)g.tau * kLog2E;
    v8i ones8, ones4;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        ones8[q] = 0x38383838;                 // E4M3 1.0
        ones4[q] = q < 4 ? 0x22222222 : 0;     // E2M1 1.0
    }

    // ================= fp8 phase: hi blocks =================
    const int32_t* hi_list = reinterpret_cast<const int32_t*>(ws + a.L.hi) + qtile * (uint64_t)g.n_hi;
    for (int jj = 0; jj < g.n_hi; ++jj) {
        const int kb = hi_list[jj];
        const uint64_t ktile = (uint64_t)bh * nb + kb;
        const uint8_t* ksrc = ws + a.L.kb + ktile * (DA2_TILE * DA2_DPAD * 2);
        const uint8_t* vsrc = ws + a.L.v8t + ktile * (DA2_DPAD * DA2_TILE);
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int ci = tid + kThreads * it;
            const int row = ci >> 4, c16 = ci & 15;
            const uint4 kx = *reinterpret_cast<const uint4*>(ksrc + ci * 16);
            *reinterpret_cast<uint4*>(kt + row * 256 + ((c16 ^ swz_k8(row)) << 4)) = kx;
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int ci = tid + kThreads * it;
            const int row = ci >> 3, c16 = ci & 7;
            const uint4 vx = *reinterpret_cast<const uint4*>(vsrc + ci * 16);
            *reinterpret_cast<uint4*>(vt + row * 128 + ((c16 ^ swz_v8(row)) << 4)) = vx;
        }
        __syncthreads();
        const int e_k8 = (int)e8[eplane + ktile] - 127;
        const int e_v8 = (int)e8[2 * eplane + ktile] - 127;
        const float cs = ldexpf(c_lo, e_q8 + e_k8);
        const bool full = block_full(g, kb);
        const BlockPos kp = block_pos(g, kb);

        v4f s[2][8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int srow = slot_fp8(t, r);
            const int sw = swz_k8(srow);
            v8bf kop[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                kop[kk] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(kt + srow * 256 + (((4 * kk + g4) ^ sw) << 4)));
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                v4f d = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kk], qbop[u][kk], d, 0, 0, 0);
                s[u][t] = d;
            }
        }
        v8i pop[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float tmax = -__builtin_huge_valf();
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x = s[u][t][e] * cs;
                    if (!full && !slot_real(g, kp, slot_fp8(t, 4 * g4 + e))) x = -__builtin_huge_valf();
                    s[u][t][e] = x;
                    tmax = fmaxf(tmax, x);
                }
            tmax = wave_max_4groups(tmax);
            const float mnew = fmaxf(m[u], ceilf(tmax));
            if (mnew > m[u]) {
                const float f = exp2f(m[u] - mnew);
#pragma unroll
                for (int ct = 0; ct < 8; ++ct) acc[u][ct] *= f;
                lsum[u] *= f;
                m[u] = mnew;
            }
            const float off = 8.0f - m[u];
#pragma unroll
            for (int t = 0; t < 8; ++t)
                pop[u][t] = (int)pack_fp8x4(__builtin_amdgcn_exp2f(s[u][t][0] + off), __builtin_amdgcn_exp2f(s[u][t][1] + off),
                                            __builtin_amdgcn_exp2f(s[u][t][2] + off), __builtin_amdgcn_exp2f(s[u][t][3] + off));
        }
        const int vscale = e_v8 + 127;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const int c = 16 * ct + r;
            const int sw = swz_v8(c);
            const v8i vop = load_lds_pair(vt, c * 128 + ((g4 ^ sw) << 4), c * 128 + (((4 + g4) ^ sw) << 4));
#pragma unroll
            for (int u = 0; u < 2; ++u)
                acc[u][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vop, pop[u], acc[u][ct], kFmtFp8, kFmtFp8,
                                                                             0, vscale, 0, 127);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
            lsum[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones8, pop[u], lsum[u], kFmtFp8, kFmtFp8, 0, 127, 0, 127);
    }

    // ================= MXFP4 phase: lo blocks =================
    const int32_t* lo_list = reinterpret_cast<const int32_t*>(ws + a.L.lo) + qtile * (uint64_t)g.n_lo;
    for (int jj = 0; jj < g.n_lo; ++jj) {
        const int kb = lo_list[jj];
        const uint64_t ktile = (uint64_t)bh * nb + kb;
        const uint8_t* ksrc = ws + a.L.k4 + ktile * (DA2_TILE * DA2_DPAD / 2);
        const uint8_t* vsrc = ws + a.L.v4t + ktile * (DA2_DPAD * DA2_TILE / 2);
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int ci = tid + kThreads * it;
            const int row = ci >> 2, c16 = ci & 3;
            const uint4 kx = *reinterpret_cast<const uint4*>(ksrc + ci * 16);
            const uint4 vx = *reinterpret_cast<const uint4*>(vsrc + ci * 16);
            *reinterpret_cast<uint4*>(kt + row * 64 + ((c16 ^ swz_k4(row)) << 4)) = kx;
            *reinterpret_cast<uint4*>(vt + row * 64 + ((c16 ^ swz_v4(row)) << 4)) = vx;
        }
        if (tid < 32) {
            *reinterpret_cast<uint4*>(ks4 + tid * 16) =
                *reinterpret_cast<const uint4*>(ws + a.L.sk4 + ktile * (DA2_TILE * 4) + tid * 16);
        } else if (tid < 64) {
            *reinterpret_cast<uint4*>(vs4 + (tid - 32) * 16) =
                *reinterpret_cast<const uint4*>(ws + a.L.sv4t + ktile * (DA2_DPAD * 4) + (tid - 32) * 16);
        }
        __syncthreads();
        const bool full = block_full(g, kb);
        const BlockPos kp = block_pos(g, kb);

        v4f s[2][8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int srow = slot_fp4(t, r);
            const v8i kop = load_lds_one(kt, srow * 64 + ((g4 ^ swz_k4(srow)) << 4));
            const int ksc = ks4[srow * 4 + g4];
#pragma unroll
            for (int u = 0; u < 2; ++u)
                s[u][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop, q4op[u], (v4f){0.f, 0.f, 0.f, 0.f},
                                                                          kFmtFp4, kFmtFp4, 0, ksc, 0, q4sc[u]);
        }
        v8i pop[2];
        int psc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float gmax = -__builtin_huge_valf();
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x = s[u][t][e] * c_lo;
                    if (!full && !slot_real(g, kp, slot_fp4(t, 4 * g4 + e))) x = -__builtin_huge_valf();
                    s[u][t][e] = x;
                    gmax = fmaxf(gmax, x);
                }
            const float tmax = wave_max_4groups(gmax);
            const float mnew = fmaxf(m[u], ceilf(tmax));
            if (mnew > m[u]) {
                const float f = exp2f(m[u] - mnew);
#pragma unroll
                for (int ct = 0; ct < 8; ++ct) acc[u][ct] *= f;
                lsum[u] *= f;
                m[u] = mnew;
            }
            // MX group of P = this lane's 32 keys: scale 2^F with F the smallest
            // integer such that 2^gmax <= 6 * 2^F; codes RNE(2^(x - F)).
            const bool any = gmax > -__builtin_huge_valf();
            const float F = any ? ceilf(gmax - kLog2Six) : 0.0f;
            const float negF = -F;
            float pv[32];
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) pv[4 * t + e] = __builtin_amdgcn_exp2f(s[u][t][e] + negF);
            pop[u][0] = (int)pack_fp4x8(pv);
            pop[u][1] = (int)pack_fp4x8(pv + 8);
            pop[u][2] = (int)pack_fp4x8(pv + 16);
            pop[u][3] = (int)pack_fp4x8(pv + 24);
            pop[u][4] = 0; pop[u][5] = 0; pop[u][6] = 0; pop[u][7] = 0;
            const int sc = any ? (int)F - (int)m[u] + 8 + 127 : 0;
            psc[u] = min(254, max(0, sc));
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const int c = 16 * ct + r;
            const v8i vop = load_lds_one(vt, c * 64 + ((g4 ^ swz_v4(c)) << 4));
            const int vsc = vs4[c * 4 + g4];
#pragma unroll
            for (int u = 0; u < 2; ++u)
                acc[u][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vop, pop[u], acc[u][ct], kFmtFp4, kFmtFp4,
                                                                             0, vsc, 0, psc[u]);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
            lsum[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones4, pop[u], lsum[u], kFmtFp4, kFmtFp4, 0, 127, 0, psc[u]);
    }

    // ================= epilogue: O = acc / l, back to raster order =================
    const BlockPos qp = block_pos(g, qb);
    const int b = bh / g.heads;
    const int h = bh - b * g.heads;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int qs = 32 * w + 16 * u + r;
        const int64_t n = slot_raster(g, qp, qs);
        if (n < 0) continue;
        const float inv = 1.0f / lsum[u][0];
        const int64_t rowoff = (int64_t)b * g.stride_b + (int64_t)h * g.stride_h + n * g.stride_n;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const int c = 16 * ct + 4 * g4;
            if (c >= g.head_dim) continue;
            const float o0 = acc[u][ct][0] * inv, o1 = acc[u][ct][1] * inv;
            const float o2 = acc[u][ct][2] * inv, o3 = acc[u][ct][3] * inv;
            if (a.out_fp32) {
                *reinterpret_cast<float4*>(static_cast<float*>(a.out) + rowoff + c) = make_float4(o0, o1, o2, o3);
            } else {
                uint2 p;
                p.x = f32_to_bf16_rne(o0) | (f32_to_bf16_rne(o1) << 16);
                p.y = f32_to_bf16_rne(o2) | (f32_to_bf16_rne(o3) << 16);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + rowoff + c) = p;
            }
        }
    }
}

hipError_t launch_attention(const Geo& g, const Layout& L, const void* ws, void* out, int out_fp32,
                            hipStream_t stream) {
    AttnArgs a;
    a.g = g;
    a.ws = static_cast<const uint8_t*>(ws);
    a.L = L;
    a.out = out;
    a.out_fp32 = out_fp32;
    hipLaunchKernelGGL(attn_kernel, dim3(g.n_blocks, g.bh), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace da2
