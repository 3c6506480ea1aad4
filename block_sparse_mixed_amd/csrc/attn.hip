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
//   The query block's key tiles (hi list, then lo list) stream through three
//   LDS buffers filled by direct global->LDS DMA two tiles ahead, so one
//   barrier per tile is the only synchronisation. Per key tile every wave runs
//     S^T = K . Q^T        fp8 phase: V_MFMA_F32_16X16X32_BF16 on the E4M3
//                          values decoded to bf16 (exact);
//                          MXFP4 phase: V_MFMA_SCALE_F32_16X16X128_F8F6F4
//     softmax (base 2, integer running max, lane-local rescale)
//     O^T += V^T . P^T     scaled f8f6f4 MFMAs (E4M3 or E2M1 operands), plus
//                          one with an all-ones A that yields the row sum
//                          l = sum P~ in the same lanes as O.
//   The QK^T of the next tile is issued in the same instruction stream as the
//   softmax of the current one, so the MFMA pipe works while the VALU
//   exponentiates. Padded key slots are excluded by starting the QK^T
//   accumulator at a per-slot bias (0 or -inf) that rides along with the tile.
//
//   Computing S transposed makes each lane hold 32 keys of one query, which
//   is exactly the B-operand layout of the PV product: P never leaves the
//   lane, the MXFP4 group of P is the lane's own 32 values, and the max
//   reduction needs two cross-lane steps (xor 16, xor 32).
//
//   The fp8 phase's QK^T runs on bf16 MFMAs because the f8f6f4 MFMA keeps only
//   about 12 bits below its largest product when it sums fp8 products: with
//   outlier channels the scores move by ~1e-2 (log2 units), enough to flip the
//   rounding of many P codes. Its PV product stays fp8: nothing is decided
//   from its rounding.
//
// Operand layouts (measured on gfx950): a 16x16x128 fp8 operand lane l holds
// row l%16 and bytes j -> k = 64*(j/16) + 16*(l/16) + j%16; an fp4 operand
// lane l holds row l%16 and nibble j -> k = 32*(l/16) + j; the E8M0 scale of
// lane l belongs to (row l%16, k-block l/16); D lane l element e is
// D[4*(l/16) + e][l%16]. A 16x16x32 bf16 MFMA only needs A and B to share
// their lane/k assignment. The key slot fed to A-row r of key tile t is chosen
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
constexpr int kHi = 0, kLo = 1, kNone = 2;

// LDS buffer layout (bytes). fp8 phase: bf16 K [128][256] | E4M3 V^T [128][128];
// MXFP4 phase: E2M1 K [128][64] | E2M1 V^T [128][64] | K scales [128][4] |
// V scales [128][4]; both: bias f32 [128] at kBias.
constexpr int kHiK = 0, kHiV = 32768;
constexpr int kLoK = 0, kLoV = 8192, kLoS = 16384;
constexpr int kBias = 49152;
constexpr int kBufBytes = kBias + 512;
constexpr int kNumBuf = 3;

// LDS swizzles (16-byte chunk index XOR a row function) so that the eight
// lanes served together by a 128-bit LDS read hit distinct banks.
__device__ __forceinline__ int swz_k8(int s) { return (s & 3) | ((s >> 2) & 4); }
__device__ __forceinline__ int swz_v8(int c) { return c & 7; }
__device__ __forceinline__ int swz_k4(int s) { return ((s >> 1) & 1) | ((s >> 4) & 2); }
__device__ __forceinline__ int swz_v4(int c) { return (c >> 1) & 3; }

__device__ __forceinline__ int slot_fp8(int t, int r) { return 64 * (t >> 2) + 16 * (r >> 2) + 4 * (t & 3) + (r & 3); }
__device__ __forceinline__ int slot_fp4(int t, int r) { return 32 * (r >> 2) + 4 * t + (r & 3); }

__device__ __forceinline__ void dma16(const void* gsrc, uint8_t* ldst) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                     (__attribute__((address_space(3))) void*)ldst, 16, 0, 0);
}

struct Tile {
    const uint8_t* k;      // bf16 K (fp8 phase) or E2M1 K
    const uint8_t* v;      // E4M3 V^T or E2M1 V^T
    const uint8_t* ks;     // E2M1 K scales (MXFP4 phase)
    const uint8_t* vs;     // E2M1 V scales (MXFP4 phase)
    const float* bias;     // per-slot 0 / -inf
    int e_k, e_v;          // fp8 block exponents (fp8 phase)
};

// Each wave moves whole 1 KiB rows of 64 x 16 bytes; lane l lands at row + 16 l.
// The gather offsets apply the LDS swizzle; for every row they reduce to a
// per-lane constant, XORed with a row-uniform bit (checked exhaustively
// against the swizzle functions above when they were derived).
struct DmaOffsets {
    uint32_t k8, k8x, v8, k4, k4x, v4;
};

__device__ __forceinline__ DmaOffsets dma_offsets(int lane) {
    DmaOffsets o;
    o.k8 = ((lane >> 4) << 8) + (((lane & 15) ^ ((lane >> 4) & 3)) << 4);
    o.k8x = o.k8 ^ 64u;
    o.v8 = ((lane >> 3) << 7) + (((lane & 7) ^ (lane >> 3)) << 4);
    o.k4 = ((lane >> 2) << 6) + (((lane & 3) ^ ((lane >> 3) & 1)) << 4);
    o.k4x = o.k4 ^ 32u;
    o.v4 = ((lane >> 2) << 6) + (((lane & 3) ^ ((lane >> 3) & 3)) << 4);
    return o;
}

__device__ __forceinline__ void dma_tile_hi(const Tile& t, uint8_t* buf, int w, int lane, const DmaOffsets& o) {
    // 32 KiB bf16 K (rows 0..31), 16 KiB V (rows 32..47), 512 B bias (half a row)
#pragma unroll
    for (int n = 0; n < 12; ++n) {
        const int wr = w * 12 + n;
        if (wr < 32)
            dma16(t.k + wr * 1024 + ((wr & 4) ? o.k8x : o.k8), buf + kHiK + wr * 1024);
        else
            dma16(t.v + (wr - 32) * 1024 + o.v8, buf + kHiV + (wr - 32) * 1024);
    }
    if (w == 0 && lane < 32) dma16(reinterpret_cast<const uint8_t*>(t.bias) + lane * 16, buf + kBias);
}

__device__ __forceinline__ void dma_tile_lo(const Tile& t, uint8_t* buf, int w, int lane, const DmaOffsets& o) {
    // 8 KiB K (rows 0..7), 8 KiB V (rows 8..15), scales 2 x 512 B, bias
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int wr = w + 4 * n;
        if (wr < 8)
            dma16(t.k + wr * 1024 + ((wr & 2) ? o.k4x : o.k4), buf + kLoK + wr * 1024);
        else
            dma16(t.v + (wr - 8) * 1024 + o.v4, buf + kLoV + (wr - 8) * 1024);
    }
    if (w == 1) dma16(lane < 32 ? t.ks + lane * 16 : t.vs + (lane - 32) * 16, buf + kLoS);
    if (w == 2 && lane < 32) dma16(reinterpret_cast<const uint8_t*>(t.bias) + lane * 16, buf + kBias);
}

struct WaveState {
    v8bf qb[2][4];         // bf16 Q operands per query tile and k-step
    v8i q4[2];             // E2M1 Q operands
    int q4s[2];            // their E8M0 scales
    v4f acc[2][8];         // O^T: [u][channel tile]; lane holds channels 16ct + 4g + e of query r
    v4f lsum[2];           // row sums (all four elements equal)
    float m[2];            // running integer max (log2 units)
    float c_lo;            // tau * log2(e)
    float c_hi_q;          // tau * log2(e) * 2^e_q8
};

// K operand of key sub-tile t for the QK^T of phase PH, read from LDS.
struct KOp {
    v8bf b[4];     // fp8 phase: bf16, one per k-step
    v8i f;         // MXFP4 phase: E2M1 codes (4 dwords used)
    v4f bias;
    int sc;        // MXFP4 phase: E8M0 scale
};

template <int PH>
__device__ __forceinline__ void load_kop(KOp& o, const uint8_t* buf, int t, int r, int g4) {
    const float* bias = reinterpret_cast<const float*>(buf + kBias);
    if constexpr (PH == kHi) {
        const int srow = slot_fp8(t, r);
        const int sw = swz_k8(srow);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            o.b[kk] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(buf + kHiK + srow * 256 + (((4 * kk + g4) ^ sw) << 4)));
        o.bias = *reinterpret_cast<const v4f*>(bias + slot_fp8(t, 4 * g4));
    } else {
        const int srow = slot_fp4(t, r);
        const uint4 x = *reinterpret_cast<const uint4*>(buf + kLoK + srow * 64 + ((g4 ^ swz_k4(srow)) << 4));
        o.f[0] = (int)x.x; o.f[1] = (int)x.y; o.f[2] = (int)x.z; o.f[3] = (int)x.w;
        o.f[4] = 0; o.f[5] = 0; o.f[6] = 0; o.f[7] = 0;
        o.sc = buf[kLoS + srow * 4 + g4];
        o.bias = *reinterpret_cast<const v4f*>(bias + slot_fp4(t, 4 * g4));
    }
}

template <int PH>
__device__ __forceinline__ void qk_sub(const WaveState& st, const KOp& o, v4f (&s)[2][8], int t) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if constexpr (PH == kHi) {
            v4f d = o.bias;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.b[kk], st.qb[u][kk], d, 0, 0, 0);
            s[u][t] = d;
        } else {
            s[u][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.f, st.q4[u], o.bias, kFmtFp4, kFmtFp4, 0, o.sc, 0,
                                                                      st.q4s[u]);
        }
    }
}

// S^T = K . Q^T for a whole key tile (used before the pipeline starts).
template <int PH>
__device__ __forceinline__ void qk(const WaveState& st, const uint8_t* buf, v4f (&s)[2][8], int r, int g4) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        KOp o;
        load_kop<PH>(o, buf, t, r, g4);
        qk_sub<PH>(st, o, s, t);
    }
}

__device__ __forceinline__ float max32(const v4f (&s)[8]) {
    float a = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
#pragma unroll
    for (int t = 1; t < 8; ++t) a = fmaxf(fmaxf(a, s[t][0]), fmaxf(fmaxf(s[t][1], s[t][2]), s[t][3]));
    return a;
}

__device__ __forceinline__ float cross4max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// One pipelined step over the current tile (phase PC, scores s_cur, LDS
// buffer cur) and the next tile (phase PN, LDS buffer nxt):
//   1. row maxima of the current scores, new running max, MX group scales;
//   2. for each key sub-tile t: the next tile's QK^T MFMAs for t next to the
//      exponentials and conversions of the current tile's sub-tile t;
//   3. rescale (rare), then O^T += V^T P^T and l += 1 P^T for the current tile.
template <int PC, int PN>
__device__ __forceinline__ void step(WaveState& st, const uint8_t* cur, const uint8_t* nxt, const v4f (&sc)[2][8],
                                     v4f (&sn)[2][8], int e_k, int e_v, int r, int g4) {
    const float cs = PC == kHi ? ldexpf(st.c_hi_q, e_k) : st.c_lo;
    float mnew[2], off[2];
    int psc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float gmax = max32(sc[u]);                  // this lane's 32 keys (raw scores)
        const float tmax = cross4max(gmax) * cs;
        mnew[u] = fmaxf(st.m[u], ceilf(tmax));
        if constexpr (PC == kHi) {
            off[u] = 8.0f - mnew[u];
            psc[u] = 127;
        } else {
            // MX group of P = this lane's 32 keys: scale 2^F, F the smallest
            // integer with 2^(gmax cs) <= 6 * 2^F; codes RNE(2^(x - F)).
            const bool any = gmax > -__builtin_huge_valf();
            const float F = any ? ceilf(gmax * cs - kLog2Six) : 0.0f;
            off[u] = -F;
            const int scl = any ? (int)F - (int)mnew[u] + 8 + 127 : 0;
            psc[u] = min(254, max(0, scl));
        }
    }
    // rescale when the running max grew (rare: tiles arrive best-ranked first);
    // done before the exponentials so that nothing gets sunk below a branch
    if (mnew[0] > st.m[0] || mnew[1] > st.m[1]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const float f = exp2f(st.m[u] - mnew[u]);
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) st.acc[u][ct] *= f;
            st.lsum[u] *= f;
        }
    }
    st.m[0] = mnew[0];
    st.m[1] = mnew[1];
    v8i pop[2];
    KOp ko[2];
    if constexpr (PN != kNone) load_kop<PN>(ko[0], nxt, 0, r, g4);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PN != kNone) {
            if (t + 1 < 8) load_kop<PN>(ko[(t + 1) & 1], nxt, t + 1, r, g4);
            qk_sub<PN>(st, ko[t & 1], sn, t);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if constexpr (PC == kHi) {
                pop[u][t] = (int)pack_fp8x4(__builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][t][0], cs, off[u])),
                                            __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][t][1], cs, off[u])),
                                            __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][t][2], cs, off[u])),
                                            __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][t][3], cs, off[u])));
            } else {
                // two E2M1 codes per conversion; a dword holds sub-tiles t and t+1
                uint32_t wv = (t & 1) ? (uint32_t)pop[u][t >> 1] : 0u;
                const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][t][0], cs, off[u]));
                const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][t][1], cs, off[u]));
                const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][t][2], cs, off[u]));
                const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][t][3], cs, off[u]));
                if (t & 1) {
                    wv = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wv, e0, e1, 1.0f, 2);
                    wv = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wv, e2, e3, 1.0f, 3);
                } else {
                    wv = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wv, e0, e1, 1.0f, 0);
                    wv = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wv, e2, e3, 1.0f, 1);
                }
                pop[u][t >> 1] = (int)wv;
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (PC == kLo) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            pop[u][4] = 0; pop[u][5] = 0; pop[u][6] = 0; pop[u][7] = 0;
        }
    }
    // O^T += V^T . P^T and l += 1 . P^T
    v8i ones;
#pragma unroll
    for (int q = 0; q < 8; ++q) ones[q] = PC == kHi ? 0x38383838 : (q < 4 ? 0x22222222 : 0);
    constexpr int fmt = PC == kHi ? kFmtFp8 : kFmtFp4;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
        const int c = 16 * ct + r;
        v8i vop;
        int vsc;
        if constexpr (PC == kHi) {
            const int sw = swz_v8(c);
            const uint4 x = *reinterpret_cast<const uint4*>(cur + kHiV + c * 128 + ((g4 ^ sw) << 4));
            const uint4 y = *reinterpret_cast<const uint4*>(cur + kHiV + c * 128 + (((4 + g4) ^ sw) << 4));
            vop[0] = (int)x.x; vop[1] = (int)x.y; vop[2] = (int)x.z; vop[3] = (int)x.w;
            vop[4] = (int)y.x; vop[5] = (int)y.y; vop[6] = (int)y.z; vop[7] = (int)y.w;
            vsc = e_v + 127;
        } else {
            const uint4 x = *reinterpret_cast<const uint4*>(cur + kLoV + c * 64 + ((g4 ^ swz_v4(c)) << 4));
            vop[0] = (int)x.x; vop[1] = (int)x.y; vop[2] = (int)x.z; vop[3] = (int)x.w;
            vop[4] = 0; vop[5] = 0; vop[6] = 0; vop[7] = 0;
            vsc = cur[kLoS + 512 + c * 4 + g4];
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
            st.acc[u][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vop, pop[u], st.acc[u][ct], fmt, fmt, 0, vsc, 0,
                                                                             psc[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
        st.lsum[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pop[u], st.lsum[u], fmt, fmt, 0, 127, 0, psc[u]);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// The key tile at position idx of the query block's list (hi blocks first).
__device__ __forceinline__ Tile tile_at(const AttnArgs& a, int bh, int qb, int idx) {
    const Geo& g = a.g;
    const uint8_t* ws = a.ws;
    const uint64_t qtile = (uint64_t)bh * g.n_blocks + qb;
    Tile t;
    int kb;
    if (idx < g.n_hi) {
        kb = reinterpret_cast<const int32_t*>(ws + a.L.hi)[qtile * g.n_hi + idx];
        const uint64_t kt = (uint64_t)bh * g.n_blocks + kb;
        t.k = ws + a.L.kb + kt * (DA2_TILE * DA2_DPAD * 2);
        t.v = ws + a.L.v8t + kt * (DA2_DPAD * DA2_TILE);
        t.ks = nullptr;
        t.vs = nullptr;
        const uint64_t plane = (uint64_t)g.bh * g.n_blocks;
        t.e_k = (int)ws[a.L.e8 + plane + kt] - 127;
        t.e_v = (int)ws[a.L.e8 + 2 * plane + kt] - 127;
    } else {
        kb = reinterpret_cast<const int32_t*>(ws + a.L.lo)[qtile * g.n_lo + (idx - g.n_hi)];
        const uint64_t kt = (uint64_t)bh * g.n_blocks + kb;
        t.k = ws + a.L.k4 + kt * (DA2_TILE * DA2_DPAD / 2);
        t.v = ws + a.L.v4t + kt * (DA2_DPAD * DA2_TILE / 2);
        t.ks = ws + a.L.sk4 + kt * (DA2_TILE * 4);
        t.vs = ws + a.L.sv4t + kt * (DA2_DPAD * 4);
        t.e_k = 0;
        t.e_v = 0;
    }
    t.bias = reinterpret_cast<const float*>(ws + a.L.bias) + (uint64_t)kb * DA2_TILE;
    return t;
}

__device__ __forceinline__ void dma_tile(const AttnArgs& a, const Tile& t, int idx, uint8_t* buf, int w, int lane,
                                         const DmaOffsets& o) {
    if (idx < a.g.n_hi)
        dma_tile_hi(t, buf, w, lane, o);
    else
        dma_tile_lo(t, buf, w, lane, o);
}

}  // namespace

__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
    const Geo& g = a.g;
    const int nb = g.n_blocks;
    // XCD-aware order: consecutive workgroups of one XCD take consecutive
    // query blocks of one head, so their key tiles meet in that XCD's L2.
    const int total = g.bh * nb;
    const int xcd = blockIdx.x & 7, k8 = blockIdx.x >> 3;
    const int per = total >> 3, rem = total & 7;
    const int logical = xcd * per + min(xcd, rem) + k8;
    const int bh = logical / nb;
    const int qb = logical - bh * nb;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r = lane & 15;
    const int g4 = lane >> 4;

    __shared__ __align__(16) uint8_t lds[kNumBuf * kBufBytes];

    const uint8_t* ws = a.ws;
    const uint64_t qtile = (uint64_t)bh * nb + qb;
    const int n_tiles = g.n_hi + g.n_lo;

    const DmaOffsets doff = dma_offsets(lane);
    // start the first two tiles' DMA before touching Q
    const Tile t0 = tile_at(a, bh, qb, 0);
    dma_tile(a, t0, 0, lds, w, lane, doff);
    Tile t1 = t0;
    if (n_tiles > 1) {
        t1 = tile_at(a, bh, qb, 1);
        dma_tile(a, t1, 1, lds + kBufBytes, w, lane, doff);
    }

    WaveState st;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int qs = 32 * w + 16 * u + r;
        const uint8_t* rowb = ws + a.L.qb + (qtile * (DA2_TILE * DA2_DPAD) + qs * DA2_DPAD) * 2;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            st.qb[u][kk] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(rowb + 64 * kk + 16 * g4));
        const uint8_t* row4 = ws + a.L.q4 + qtile * (DA2_TILE * DA2_DPAD / 2) + qs * (DA2_DPAD / 2);
        const uint4 x4 = *reinterpret_cast<const uint4*>(row4 + 16 * g4);
        st.q4[u][0] = (int)x4.x; st.q4[u][1] = (int)x4.y; st.q4[u][2] = (int)x4.z; st.q4[u][3] = (int)x4.w;
        st.q4[u][4] = 0; st.q4[u][5] = 0; st.q4[u][6] = 0; st.q4[u][7] = 0;
        st.q4s[u] = (int)ws[a.L.sq4 + qtile * (DA2_TILE * DA2_DPAD / 32) + qs * (DA2_DPAD / 32) + g4];
        st.m[u] = -__builtin_huge_valf();
        st.lsum[u] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) st.acc[u][ct] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
    st.c_lo = (float)g.tau * kLog2E;
    st.c_hi_q = ldexpf(st.c_lo, (int)ws[a.L.e8 + qtile] - 127);

    v4f sA[2][8], sB[2][8];
    __builtin_amdgcn_s_waitcnt(0);     // tiles 0 and 1 and the Q operands
    __syncthreads();
    if (g.n_hi > 0)
        qk<kHi>(st, lds, sA, r, g4);
    else
        qk<kLo>(st, lds, sA, r, g4);

    // Tile idx lives in buffer idx % 3; its scores are in sA when it is the
    // current tile. Each step first issues the DMA of tile idx + 2 into the
    // buffer of tile idx - 1, whose readers all passed the previous barrier.
    Tile cur = t0, nxt = t1;
    int idx = 0;
    auto issue_next = [&]() {
        Tile t2 = nxt;
        if (idx + 2 < n_tiles) {
            t2 = tile_at(a, bh, qb, idx + 2);
            dma_tile(a, t2, idx + 2, lds + ((idx + 2) % 3) * kBufBytes, w, lane, doff);
        }
        return t2;
    };
    auto finish = [&](const Tile& t2) {
        cur = nxt;
        nxt = t2;
        ++idx;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    // fp8 phase, pipelined while the next tile is fp8 too
    for (; idx + 1 < g.n_hi; ) {
        const Tile t2 = issue_next();
        step<kHi, kHi>(st, lds + (idx % 3) * kBufBytes, lds + ((idx + 1) % 3) * kBufBytes, sA, sB, cur.e_k, cur.e_v, r, g4);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < 8; ++t) sA[u][t] = sB[u][t];
        finish(t2);
    }
    if (g.n_hi > 0) {
        // last fp8 tile, then the first MXFP4 tile's QK^T on its own
        const Tile t2 = issue_next();
        step<kHi, kNone>(st, lds + (idx % 3) * kBufBytes, lds, sA, sB, cur.e_k, cur.e_v, r, g4);
        finish(t2);
        if (idx < n_tiles) qk<kLo>(st, lds + (idx % 3) * kBufBytes, sA, r, g4);
    }
    // MXFP4 phase
    for (; idx + 1 < n_tiles; ) {
        const Tile t2 = issue_next();
        step<kLo, kLo>(st, lds + (idx % 3) * kBufBytes, lds + ((idx + 1) % 3) * kBufBytes, sA, sB, 0, 0, r, g4);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < 8; ++t) sA[u][t] = sB[u][t];
        finish(t2);
    }
    if (idx < n_tiles) {
        step<kLo, kNone>(st, lds + (idx % 3) * kBufBytes, lds, sA, sB, 0, 0, r, g4);
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
        const float inv = 1.0f / st.lsum[u][0];
        const int64_t rowoff = (int64_t)b * g.stride_b + (int64_t)h * g.stride_h + n * g.stride_n;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const int c = 16 * ct + 4 * g4;
            if (c >= g.head_dim) continue;
            const float o0 = st.acc[u][ct][0] * inv, o1 = st.acc[u][ct][1] * inv;
            const float o2 = st.acc[u][ct][2] * inv, o3 = st.acc[u][ct][3] * inv;
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
    const int total = g.bh * g.n_blocks;
    return launch_kernel(attn_kernel, dim3(total), dim3(kThreads), 0, stream, a);
}

}  // namespace da2
