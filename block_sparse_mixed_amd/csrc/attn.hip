// K3: block-sparse flash attention with an fp8 phase and an MXFP4 phase.
//
// [DraftAttention2 (arXiv 2609.32628), abstract]: one attention kernel with
// precision-specific phases that share data movement, the softmax statistics
// and the output accumulator; 8-bit compute on the top-ranked blocks, 4-bit on
// the other retained blocks, nothing on skipped blocks. [DraftAttention
// (arXiv 2505.14708), abstract]: outputs return to the original token order.
//
// Work decomposition (gfx950, wave64):
//   one workgroup = one query block (128 slots) of one (batch, head), eight
//   waves in two teams of four. Wave w%4 of either team owns query slots
//   32(w%4) .. +32: lane l works for query l%32, the lanes l and l+32 (halves
//   h = 0, 1) for the same query. The query block's key tiles run as two
//   sections, the hi list and then the lo list (each best-ranked first), so
//   that every loop body has a single precision. Within a section the tiles
//   alternate between the teams: team 0 takes tiles 0, 2, 4, ..., team 1
//   tiles 1, 3, 5, ...
//   Time runs in phases separated by workgroup barriers. In phase p the team
//   owning tile p runs its matrix work, PV of tile p-2 and QK^T of tile p,
//   while the other team runs the softmax of tile p-1. The two waves sharing
//   a SIMD are therefore always in opposite halves of their work: one feeds
//   the matrix pipe while the other exponentiates.
//     S^T = K . Q^T        fp8 tiles: V_MFMA_F32_32X32X16_BF16 on the E4M3
//                          values widened to bf16 (exact): Q once per
//                          workgroup into LDS, K in registers from the E4M3
//                          codes in LDS;
//                          MXFP4 tiles: V_MFMA_SCALE_F32_32X32X64_F8F6F4
//     softmax (base 2, integer running max per team, lane-local rescale)
//     O^T += V^T . P^T     scaled 32x32x64 f8f6f4 MFMAs (E4M3 or E2M1
//                          operands), plus one with an all-ones A that yields
//                          the row sum l = sum P~ in the same lanes as O.
//   The 32x32 shapes issue half the MFMA instructions of the 16x16 ones for
//   the same work, and on gfx950 an MFMA costs about the same issue time at
//   either size: issue, not the matrix pipe, bounds this kernel.
//   The query block's Q operands (bf16 and E2M1) sit in LDS for the whole
//   kernel. K and V^T of a tile travel by direct global->LDS DMA into
//   separate two-slot pools: K of tile p+1 and V^T of tile p-1 are issued
//   during phase p by the team running the softmax, between its maximum and
//   its exponentials (a DMA instruction holds only the wave that issues it,
//   so the matrix wave sharing its SIMD keeps issuing, and the
//   exponentials hide the DMA latency). The tile list entries each team needs travel in scalar
//   registers, read from LDS one trip ahead. At the end the teams' (max, sum,
//   accumulator) triples merge exactly: their maxima are integers, so the
//   rescale factors are powers of two. Padded key slots are excluded by
//   starting the QK^T accumulator at a per-slot bias (0 or -inf) that travels
//   with K.
//
//   Computing S transposed makes each lane hold 64 keys of one query (the
//   other 64 in its partner lane), which is exactly the B-operand layout of
//   the PV product: P never leaves the lane, each MXFP4 group of P is 32 of
//   the lane's own values, and the max reduction needs one cross-lane step.
//
//   Register budget: two waves per SIMD leave 256 registers per wave, of
//   which the accumulator takes 64 and the scores another 64. The code is
//   shaped so the allocator needs no copies or spills in the loops: static
//   slot parity, no precision branches and no per-phase conditions inside a
//   loop body, values derived from the lane index recomputed where used,
//   E2M1 operands kept as four dwords, and the rare rescale done in place.
//
//   The fp8 tiles' QK^T runs on bf16 MFMAs because the f8f6f4 MFMAs (and the
//   unscaled fp8 ones) keep only about 12 bits below their largest product
//   when they sum fp8 products (tests/test_gpu_hardware_facts.py measures it):
//   with outlier channels the scores move by ~1e-2 (log2 units), enough to
//   flip the rounding of many P codes. Their PV product stays fp8: nothing is
//   decided from its rounding.
//
// Operand layouts of the 32x32 MFMAs (gfx950): A lane l holds row l%32 and B
// lane l column l%32, both for the same half h = l/32 of the k range (an E2M1
// operand: nibble i -> k = 32 h + i, whose E8M0 scale lane l supplies); the
// result D lane l element j is D[8*(j/4) + 4*h + j%4][l%32]. A and B only
// need to agree on which k each lane byte carries. The key slot fed to A row
// r of QK^T key block kb (sigma_fp8, sigma_fp4) is chosen so that the keys
// whose P a lane holds for one PV MFMA are the slots that lane's V^T operand
// reads in natural order.
#include <type_traits>
#include <utility>

#include "common.hpp"

namespace da2 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

struct AttnArgs {
    Geo g;
    const uint8_t* ws;
    Layout L;
    void* out;
    int out_fp32;
};

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kTeamWaves = kWaves / 2;
constexpr int kFmtFp8 = 0;
constexpr int kFmtFp4 = 4;
constexpr float kLog2E = 1.4426950408889634f;
constexpr float kLog2Six = 2.5849625007211562f;
constexpr int kHi = 0, kLo = 1;

// LDS: K slots [K data | bias f32[128] | E8M0 K scales [128][4]] and V slots
// [V^T data 16 KiB | E8M0 V scales [128][4]], two of each, and Q.
// fp8 tiles: K data = E4M3 [128 slots][128 B], V data = E4M3 [128 ch][128 B];
// MXFP4 tiles: K data = E2M1 [128 slots][64 B], V data = E2M1 [128 ch][64 B].
// A K slot is sized for the exchange area of the final team merge (two waves'
// accumulators), which it doubles as; the tiles use at most 16 KiB of it.
constexpr int kKBias = 32768, kKScale = 33280, kKSlot = 33792;
constexpr int kVScale = 16384, kVSlot = 16896;
// Q: bf16 [128][256 B] | E2M1 [128][64 B] | E8M0 [128][4]
constexpr int kQb = 0, kQ4 = 32768, kQs = 40960, kQBytes = 41472;
constexpr int kListBytes = 4 * DA2_MAX_BLOCKS;    // packed tile list
static_assert(2 * 65 * 64 * 4 <= kKSlot, "team merge area: two waves per K slot");

// LDS swizzles (16-byte chunk index XOR a row function) so that the sixteen
// lanes served together by a 128-bit LDS read (64 banks of 4 bytes) hit
// sixteen distinct 16-byte bank groups; each depends only on the lane's
// query or channel index, not on the step.
__device__ __forceinline__ int swz_k8f(int s) { return ((s >> 1) & 1) | (((s >> 4) & 1) << 1) | (((s >> 2) & 1) << 2); }
__device__ __forceinline__ int swz_v8(int c) { return (c >> 1) & 7; }
__device__ __forceinline__ int swz_k4(int s) { return ((s >> 2) & 1) | ((s >> 4) & 2); }
__device__ __forceinline__ int swz_v4(int c) { return (c >> 2) & 3; }

// The key slot fed to A row r (0 .. 31) of QK^T key block kb (0 .. 3). A
// 32x32 MFMA result row r sits in lane half (r / 4) % 2 at register
// 4 (r / 8) + r % 4; these maps make each lane's scores of one PV MFMA the
// keys that the PV's V^T operand holds in natural slot order in that lane.
__device__ __forceinline__ int sigma_fp8(int kb, int r) { return 32 * kb + 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }
__device__ __forceinline__ int sigma_fp4(int kb, int r) {
    return 64 * (kb >> 1) + 16 * (kb & 1) + 32 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

// Keeps an MFMA source operand alive past its last MFMA, so that the register
// allocator never gives that MFMA a destination overlapping the operand (the
// hardware still reads sources while a multi-pass MFMA writes its result).
// The asm statement reads and "rewrites" the operand, so it cannot be
// scheduled ahead of the MFMAs that read it.
template <class T>
__device__ __forceinline__ void keep(T& x) {
    asm volatile("" : "+v"(x));
}

// The lane index computed afresh where it is used: the compiler cannot hoist
// an asm statement out of a loop, so nothing lane-dependent stays live (and
// spills) across the main loop. Two ALU instructions, no memory access.
__device__ __forceinline__ int fresh_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Scheduling fence: nothing moves across it, which bounds register live ranges.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(std::integral_constant<int, i>) for i = 0 .. N-1
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ void dma16(const void* gsrc, uint8_t* ldst) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                     (__attribute__((address_space(3))) void*)ldst, 16, 0, 0);
}

// Per-lane gather offsets of a 1 KiB DMA row that apply the LDS swizzle; for
// every row they reduce to a per-lane constant, XORed with a row-uniform bit.
struct DmaOffsets {
    uint32_t v8, k4, v4, k8f;
};

__device__ __forceinline__ DmaOffsets dma_offsets(int lane) {
    DmaOffsets o;
    // E4M3 V^T rows (128 B): a DMA of channels 8i .. 8i+7 gathers with this
    // offset XOR ((i & 1) << 6)
    o.v8 = ((lane >> 3) << 7) + (((lane & 7) ^ ((lane >> 4) & 3)) << 4);
    // E2M1 K rows (64 B): a DMA of slots 16i .. 16i+15 gathers with this
    // offset XOR ((i & 2) << 4)
    o.k4 = ((lane >> 2) << 6) + (((lane & 3) ^ ((lane >> 4) & 1)) << 4);
    o.v4 = ((lane >> 2) << 6) + (((lane & 3) ^ ((lane >> 4) & 3)) << 4);
    // E4M3 K rows (128 B): chunk c of row s sits at c ^ swz_k8f(s); a DMA of
    // rows 8i .. 8i+7 gathers with this offset XOR (((i >> 1) & 1) << 5)
    o.k8f = ((lane >> 3) << 7) + (((lane & 7) ^ ((lane >> 4) & 1) ^ (((lane >> 5) & 1) << 2)) << 4);
    return o;
}

struct Tile {
    const uint8_t* k;      // E4M3 K (fp8 tile) or E2M1 K
    const uint8_t* v;      // E4M3 V^T or E2M1 V^T
    const uint8_t* ks;     // E2M1 K scales
    const uint8_t* vs;     // E2M1 V scales
    const float* bias;     // per-slot 0 / -inf
    int e_k, e_v;          // fp8 block exponents
};

// The key tile at position idx of the query block's list (hi blocks first),
// from the packed copy of the list in LDS: block index in bits 0-15, biased
// K and V fp8 exponents in bits 16-23 and 24-31.
// The packed entry is made wave-uniform (a scalar register) so that all the
// tile's address arithmetic is scalar.
template <int PH>
__device__ __forceinline__ Tile tile_from(const AttnArgs& a, const uint8_t* __restrict__ ws, int bh, int32_t entry) {
    const Geo& g = a.g;
    const uint32_t e = (uint32_t)__builtin_amdgcn_readfirstlane(entry);
    const int kb = (int)(e & 0xFFFFu);
    const uint64_t kt = (uint64_t)bh * g.n_blocks + kb;
    Tile t;
    if constexpr (PH == kHi) {
        t.k = ws + a.L.k8 + kt * (DA2_TILE * DA2_DPAD);
        t.v = ws + a.L.v8t + kt * (DA2_DPAD * DA2_TILE);
        t.ks = nullptr;
        t.vs = nullptr;
        t.e_k = (int)((e >> 16) & 0xFFu) - 127;
        t.e_v = (int)(e >> 24) - 127;
    } else {
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

// A phase's fetch, K(p+1) and V^T(p-1), is spread over the four waves of one
// team as a short list of DMA items per wave (w = the wave's index in its
// team): fp8 tiles 4 K rows, 4 V rows and the K bias; MXFP4 tiles 2 K rows,
// 2 V rows, the K scales and bias, and the V scales. A row is 1 KiB, one
// instruction over the wave's 64 lanes.
template <int PH>
constexpr int kFetchItems = PH == kHi ? 9 : 6;

// Row wr (1 KiB) of a tile's K codes, or of its V^T codes, into a slot.
template <int PH>
__device__ __forceinline__ void k_row(const Tile& t, uint8_t* slot, int wr, const DmaOffsets& o) {
    if constexpr (PH == kHi)   // 16 KiB of E4M3 K: 8 key rows per 1 KiB row
        dma16(t.k + wr * 1024 + (o.k8f ^ (((wr >> 1) & 1) << 5)), slot + wr * 1024);
    else                       // 8 KiB of E2M1 K
        dma16(t.k + wr * 1024 + (o.k4 ^ ((wr & 2) << 4)), slot + wr * 1024);
}
template <int PH>
__device__ __forceinline__ void v_row(const Tile& t, uint8_t* slot, int wr, const DmaOffsets& o) {
    if constexpr (PH == kHi)   // 16 KiB of E4M3 V^T
        dma16(t.v + wr * 1024 + (o.v8 ^ ((wr & 1) << 6)), slot + wr * 1024);
    else                       // 8 KiB of E2M1 V^T
        dma16(t.v + wr * 1024 + o.v4, slot + wr * 1024);
}
// The key-slot bias (wave 0) and, for MXFP4 tiles, the K scales (wave 1).
template <int PH>
__device__ __forceinline__ void k_extras(const Tile& t, uint8_t* slot, int w, int lane) {
    if constexpr (PH == kLo)
        if (w == 1 && lane < 32) dma16(t.ks + (uint32_t)lane * 16, slot + kKScale);
    if (w == 0 && lane < 32) dma16(reinterpret_cast<const uint8_t*>(t.bias) + (uint32_t)lane * 16, slot + kKBias);
}

template <int PH, int I>
__device__ __forceinline__ void fetch_item(const Tile& tk, uint8_t* kslot, const Tile& tv, uint8_t* vslot, int w,
                                           int lane, const DmaOffsets& o) {
    constexpr int kRows = (PH == kHi ? 16 : 8) / kTeamWaves;
    if constexpr (I < kRows) {
        k_row<PH>(tk, kslot, w + kTeamWaves * I, o);
    } else if constexpr (I < 2 * kRows) {
        v_row<PH>(tv, vslot, w + kTeamWaves * (I - kRows), o);
    } else if constexpr (I == 2 * kRows) {
        k_extras<PH>(tk, kslot, w, lane);
    } else {
        static_assert(PH == kLo && I == 2 * kRows + 1, "fetch item");
        if (w == 3 && lane < 32) dma16(tv.vs + (uint32_t)lane * 16, vslot + kVScale);   // MXFP4 V scales
    }
}

// All of a team's K items of one tile (the first tile of a section).
template <int PH>
__device__ __forceinline__ void dma_k(const Tile& t, uint8_t* slot, int w, int lane, const DmaOffsets& o) {
#pragma unroll
    for (int n = 0; n < (PH == kHi ? 16 : 8) / kTeamWaves; ++n) k_row<PH>(t, slot, w + kTeamWaves * n, o);
    k_extras<PH>(t, slot, w, lane);
}

struct WaveState {
    const uint8_t* q;      // LDS Q block
    int qs0;               // first query slot of this wave
    // O^T by channel block cb: element j holds channel 32 cb + 8 (j / 4) + 4 h
    // + j % 4 of the lane's query (h = lane / 32)
    v16f acc[4];
    v16f lsum;             // the query's row sum (all sixteen elements equal)
    float m;               // running integer max (log2 units)
    float mref;            // acc and lsum hold values relative to 2^mref
    float c_lo;            // tau * log2(e), at least FLT_MIN
    int e_q;               // fp8 block exponent of the query block
};

// A 32x32x64 MFMA operand in E2M1 occupies four registers; the builtin takes
// eight, of which the hardware reads the first four for this format. Building
// the vector at the call keeps only the four live values in registers.
__device__ __forceinline__ v8i fp4_operand(v4i x) {
    return __builtin_shufflevector(x, (v4i){0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ v4i as_v4i(const uint4& x) { return (v4i){(int)x.x, (int)x.y, (int)x.z, (int)x.w}; }

// ---- Q operands of the wave's 32 queries, read from LDS ----
// Q rows in LDS are swizzled: bf16 16-byte chunk c of query slot q sits at
// chunk c ^ (q & 15); E2M1 chunk c at c ^ ((q >> 2) & 3).
// Lane (query q, half h) feeds the bf16 MFMAs channels 32 i + 16 h .. + 15
// (two MFMAs of 8 channels per i) and the E2M1 MFMAs channels 64 c + 32 h ..
// + 31; K uses the same assignment.
struct QOps {
    v8bf qb[4][2];         // bf16 (fp8 phase): [i][e], channels 32 i + 16 h + 8 e .. + 7
    v4i q4[2];             // E2M1 (MXFP4 phase): [c], channels 64 c + 32 h .. + 31
    int q4s[2];            // their E8M0 scales
};

template <int PH>
__device__ __forceinline__ void load_q(const WaveState& st, QOps& qo, int q, int h) {
    const int qs = st.qs0 + q;                 // qs & 31 == q: qs0 is a multiple of 32
    if constexpr (PH == kHi) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                qo.qb[i][e] = __builtin_bit_cast(
                    v8bf, *reinterpret_cast<const uint4*>(st.q + kQb + qs * 256 + (((4 * i + 2 * h + e) ^ (q & 15)) << 4)));
    } else {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int chunk = 2 * c + h;
            qo.q4[c] = as_v4i(*reinterpret_cast<const uint4*>(st.q + kQ4 + qs * 64 + ((chunk ^ ((q >> 2) & 3)) << 4)));
            qo.q4s[c] = st.q[kQs + qs * 4 + chunk];
        }
    }
}

__device__ __forceinline__ v8bf widen_e4m3(uint32_t lo, uint32_t hi) {
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true);
    return (v8bf){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// ---- S^T = K . Q^T for one key tile ----
// Output s[kb] (key block kb of 32 rows): element j of lane (q, h) is the
// score of query q against the key slot the row 8 (j / 4) + 4 h + j % 4 of
// block kb was fed with, which is slot 32 kb + 16 h + j (fp8) or
// 64 (kb / 2) + 32 h + 16 (kb % 2) + j (MXFP4): see sigma_fp8 / sigma_fp4.
// The accumulator starts at the key's bias (0, or -inf for a padded slot).
template <int PH>
__device__ __forceinline__ void qk(const uint8_t* ks, QOps& qo, v16f (&s)[4], int q, int h) {
    if constexpr (PH == kHi) {
        // A row q of block kb is key slot sigma_fp8(kb, q) = 32 kb + rho(q);
        // the swizzle of that row depends on q only
        const int rho = sigma_fp8(0, q);
        const int sw = swz_k8f(rho);
        // lane base addresses of the 16-byte chunks 2 i + h, i = 0 .. 3
        const uint8_t* kp[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) kp[i] = ks + rho * 128 + (((2 * i + h) ^ sw) << 4);
        const uint8_t* bp = ks + kKBias + 64 * h;
        // the accumulators start at the bias, all read up front
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const v4f b4 = *reinterpret_cast<const v4f*>(bp + 128 * kb + 16 * e4);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[kb][4 * e4 + e] = b4[e];
            }
        // one step = (kb, i): 16 E4M3 codes, widened, feed two MFMAs; the
        // codes are read 2 - 1 steps ahead (the fence after each read keeps
        // the scheduler from sinking it towards its use)
        constexpr int R = 2;
        uint4 code[R];
#pragma unroll
        for (int t = 0; t + 1 < R; ++t) code[t] = *reinterpret_cast<const uint4*>(kp[t & 3] + 4096 * (t >> 2));
        fence();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int step = 4 * kb + i;
                if (step + R - 1 < 16) {
                    code[(step + R - 1) % R] =
                        *reinterpret_cast<const uint4*>(kp[(step + R - 1) & 3] + 4096 * ((step + R - 1) >> 2));
                    fence();
                }
                const uint4& x = code[step % R];
                v8bf kb0 = widen_e4m3(x.x, x.y);
                v8bf kb1 = widen_e4m3(x.z, x.w);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb0, qo.qb[i][0], s[kb], 0, 0, 0);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb1, qo.qb[i][1], s[kb], 0, 0, 0);
                keep(kb0);
                keep(kb1);
                fence();
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            keep(qo.qb[i][0]);
            keep(qo.qb[i][1]);
        }
    } else {
        const int rho = sigma_fp4(0, q);           // sigma_fp4(kb, q) = rho + 64 (kb / 2) + 16 (kb % 2)
        const int sw = swz_k4(rho);
        const uint8_t* kp[2];
        const uint8_t* sp[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            kp[c] = ks + rho * 64 + (((2 * c + h) ^ sw) << 4);
            sp[c] = ks + kKScale + rho * 4 + 2 * c + h;
        }
        const uint8_t* bp = ks + kKBias + 128 * h;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int off = 64 * (kb >> 1) + 16 * (kb & 1);     // slot offset of block kb's rows
            v16f d;
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const v4f b4 = *reinterpret_cast<const v4f*>(bp + 4 * off + 16 * e4);
#pragma unroll
                for (int e = 0; e < 4; ++e) d[4 * e4 + e] = b4[e];
            }
            v4i k4[2];
            int ksc[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                k4[c] = as_v4i(*reinterpret_cast<const uint4*>(kp[c] + off * 64));
                ksc[c] = sp[c][off * 4];
            }
#pragma unroll
            for (int c = 0; c < 2; ++c)
                d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(k4[c]), fp4_operand(qo.q4[c]), d, kFmtFp4,
                                                                   kFmtFp4, 0, ksc[c], 0, qo.q4s[c]);
            keep(k4[0]);
            keep(k4[1]);
            s[kb] = d;
            fence();
        }
        keep(qo.q4[0]);
        keep(qo.q4[1]);
    }
}

// x *= f, computed in x's own registers. A plain multiply on a rarely taken
// branch lets the register allocator place the product elsewhere, and the
// merge after the branch then costs a copy of the whole accumulator on the
// common path.
__device__ __forceinline__ void scale_in_place(v16f& x, float f) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        float y = x[e];
        asm("v_mul_f32 %0, %0, %1" : "+v"(y) : "v"(f));
        x[e] = y;
    }
}

// IEEE maximum (V_MAXIMUM3_F32 on gfx950). The scores are never NaN, so it
// equals the usual max here; unlike fmaxf it needs no NaN-quieting move in
// front of an MFMA result, and unlike a hand-written V_MAX3_F32 the compiler
// knows it is a plain ALU op and adds no wait states after it.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// The lane's maximum over each pair of key blocks (2n, 2n+1): four chains of
// three-input maxima, one per key block, advanced in lockstep so that no
// step waits on the step before it (one dependent chain needs a wait state
// between its steps).
__device__ __forceinline__ void block_max(const v16f (&s)[4], float (&gmax)[2]) {
    float a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = vmax3(s[k][0], s[k][1], s[k][2]);
#pragma unroll
    for (int i = 3; i + 1 < 16; i += 2)
#pragma unroll
        for (int k = 0; k < 4; ++k) a[k] = vmax3(a[k], s[k][i], s[k][i + 1]);
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = vmax(a[k], s[k][15]);
    gmax[0] = vmax(a[0], a[1]);
    gmax[1] = vmax(a[2], a[3]);
}

// Max over the two lanes l and l ^ 32 (the query's two halves of keys): the
// permlane swap exchanges two copies' halves, so the maximum of its two
// results is the pairwise maximum; no LDS traffic.
__device__ __forceinline__ float cross2max(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
}

// ---- softmax of one tile: P operands and their E8M0 scales ----
// The P codes of a tile are taken relative to the running integer max m (so
// they are the codes the oracle takes relative to the final max, shifted by
// a power of two). The accumulator and row sum are kept relative to a
// reference 2^mref instead, and the factor 2^(m - mref) rides in the P scale
// operand of the PV and row-sum MFMAs: a growing maximum costs no pass over
// the accumulator. Only when m runs more than kMaxLead above mref (or at the
// first tile, mref = -inf) is the accumulator rescaled, by an exact power of
// two, and mref moved to m.
//   P operand of PV MFMA n (keys 64 n .. 64 n + 63 of the PV order): the
// lane's scores of key blocks 2 n and 2 n + 1, in register order.
//   fetch() issues the phase's DMA. In fp8 phases it is called after the
// maximum, in MXFP4 phases after the P codes and scales; in both, the
// compiler then places the exponentials (pure, and read only in the next
// phase) after the DMA instructions, so that the exponentials hide the DMA
// latency before the phase's closing barrier. Measured slower: the DMA
// before the maximum, spread among the exponentials, or forced after them.
constexpr float kMaxLead = 64.0f;

template <int PH, class Fetch>
__device__ __forceinline__ void softmax(WaveState& st, const v16f (&s)[4], int e_k, v8i (&pop)[2], int (&psc)[2],
                                        Fetch&& fetch) {
    // fp8 tiles: the codes' product carries 2^(e_q + e_k), applied in one
    // step (no intermediate underflow) and kept at least FLT_MIN, so that a
    // padded key's -inf score stays -inf (0 * -inf would be NaN) when the
    // two blocks' magnitudes are so small that the factor underflows; the
    // real scores are then below 2^-100 in either case
    const float cs = PH == kHi ? fmaxf(ldexpf(st.c_lo, st.e_q + e_k), __FLT_MIN__) : st.c_lo;
    float gmax[2];                                       // per PV MFMA n: the lane's 32 raw scores
    block_max(s, gmax);
    const float mnew = vmax(st.m, ceilf(cross2max(vmax(gmax[0], gmax[1])) * cs));
    if (!(st.mref >= mnew - kMaxLead)) {
        const float f = exp2f(st.mref - mnew);           // 0 while mref = -inf
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) scale_in_place(st.acc[cb], f);
        scale_in_place(st.lsum, f);
        st.mref = mnew;
    }
    if constexpr (PH == kHi) fetch();
    static_for<2>([&](auto nc) __attribute__((always_inline)) {
        constexpr int n = decltype(nc)::value;
        if constexpr (PH == kHi) {
            // finite also while no key has been seen (mnew = -inf): the
            // scores are then -inf and the codes 0
            const float off = 8.0f - vmax(mnew, -__FLT_MAX__);
            static_for<8>([&](auto dc) __attribute__((always_inline)) {
                constexpr int d = decltype(dc)::value;   // bytes 4 d .. 4 d + 3
                const v16f& x = s[2 * n + (d >> 2)];
                constexpr int j = 4 * (d & 3);
                pop[n][d] = (int)pack_fp8x4(__builtin_amdgcn_exp2f(__builtin_fmaf(x[j], cs, off)),
                                            __builtin_amdgcn_exp2f(__builtin_fmaf(x[j + 1], cs, off)),
                                            __builtin_amdgcn_exp2f(__builtin_fmaf(x[j + 2], cs, off)),
                                            __builtin_amdgcn_exp2f(__builtin_fmaf(x[j + 3], cs, off)));
            });
            // 127 .. 127 + kMaxLead (127 while no key has been seen: both -inf)
            psc[n] = 127 + (int)vmax(mnew - st.mref, 0.0f);
        } else {
            // MX group of P = the lane's 32 keys of this PV MFMA: scale 2^F,
            // F the smallest integer with 2^(gmax cs) <= 6 * 2^F; codes
            // RNE(2^(x - F)).
            const bool any = gmax[n] > -__builtin_huge_valf();
            const float F = any ? ceilf(gmax[n] * cs - kLog2Six) : 0.0f;
            const float off = -F;
            static_for<4>([&](auto dc) __attribute__((always_inline)) {
                constexpr int d = decltype(dc)::value;   // nibbles 8 d .. 8 d + 7
                const v16f& x = s[2 * n + (d >> 1)];
                constexpr int j = 8 * (d & 1);
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j + e], cs, off));
                pop[n][d] = (int)pack_fp4x8(v);
            });
            const int sc = any ? (int)(F - st.mref) + 8 + 127 : 0;
            psc[n] = min(254, max(0, sc));
        }
    });
    st.m = mnew;
    if constexpr (PH == kLo) fetch();
}

// ---- O^T += V^T . P^T and l += 1 . P^T ----
// PV MFMA (n, cb): A = V^T channels 32 cb .. + 31 over keys 64 n .. + 63 in
// natural slot order. Lane (channel row q, half h) holds, for fp8, the 16
// slots 64 n + 16 h .. + 15 then 64 n + 32 + 16 h .. + 15, and for E2M1 the
// 32 slots 64 n + 32 h .. + 31: exactly the keys whose P the lane of query q
// and the same half holds (see qk).
template <int PH>
struct VOps;
template <>
struct VOps<kHi> {
    v8i v;                 // E4M3
};
template <>
struct VOps<kLo> {
    v4i v;                 // E2M1
    int sc;
};

template <int PH>
__device__ __forceinline__ void load_v(const uint8_t* vs, int n, int cb, int q, int h, VOps<PH>& o) {
    // channel 32 cb + q; its swizzle depends on q only
    if constexpr (PH == kHi) {
        const int sw = swz_v8(q);
        const uint8_t* row = vs + q * 128 + 4096 * cb;     // cb in the immediate offsets
        const uint4 x = *reinterpret_cast<const uint4*>(row + (((4 * n + h) ^ sw) << 4));
        const uint4 y = *reinterpret_cast<const uint4*>(row + (((4 * n + 2 + h) ^ sw) << 4));
        o.v = (v8i){(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    } else {
        // lane part + compile-time part, so that cb and n land in the
        // instructions' immediate offsets
        const uint8_t* row = vs + q * 64 + 2048 * cb;
        o.v = as_v4i(*reinterpret_cast<const uint4*>(row + (((2 * n + h) ^ swz_v4(q)) << 4)));
        o.sc = vs[kVScale + q * 4 + h + 128 * cb + 2 * n];
    }
}

template <int PH>
__device__ __forceinline__ void pv(WaveState& st, const uint8_t* vs, v8i (&pop)[2], const int (&psc)[2], int e_v,
                                   int q, int h) {
    constexpr int fmt = PH == kHi ? kFmtFp8 : kFmtFp4;
    constexpr int D = 3;      // 2 and 4+ measured slower in MXFP4 phases, equal in fp8 ones
    VOps<PH> o[D + 1];
    // B operand: P^T (E2M1 uses the low four dwords)
    v8i pb[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        if constexpr (PH == kHi)
            pb[n] = pop[n];
        else
            pb[n] = fp4_operand(__builtin_shufflevector(pop[n], pop[n], 0, 1, 2, 3));
    }
    const int vsc_hi = e_v + 127;
    // steps (n, cb), V^T operands read D steps ahead
#pragma unroll
    for (int t = 0; t < D; ++t) load_v<PH>(vs, t >> 2, t & 3, q, h, o[t]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        if (t + D < 8) load_v<PH>(vs, (t + D) >> 2, (t + D) & 3, q, h, o[(t + D) % (D + 1)]);
        VOps<PH>& c = o[t % (D + 1)];
        const int n = t >> 2, cb = t & 3;
        v8i va;
        int vsc;
        if constexpr (PH == kHi) {
            va = c.v;
            vsc = vsc_hi;
        } else {
            va = fp4_operand(c.v);
            vsc = c.sc;
        }
        st.acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb[n], st.acc[cb], fmt, fmt, 0, vsc, 0, psc[n]);
        keep(c.v);
        fence();
    }
    // all-ones A operand (E4M3 1.0 = 0x38, E2M1 1.0 = 0x2), built here so it
    // is never kept live (or spilled) between tiles
    int one = PH == kHi ? 0x38383838 : 0x22222222;
    asm volatile("" : "+v"(one));          // not hoisted out of the loop
    v8i ones;
#pragma unroll
    for (int w = 0; w < 8; ++w) ones[w] = (PH == kHi || w < 4) ? one : 0;
#pragma unroll
    for (int n = 0; n < 2; ++n)
        st.lsum = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pb[n], st.lsum, fmt, fmt, 0, 127, 0, psc[n]);
    keep(one);
    if constexpr (PH == kHi) {
        keep(pop[0]);
        keep(pop[1]);
    } else {
        v4i p0 = __builtin_shufflevector(pop[0], pop[0], 0, 1, 2, 3);
        v4i p1 = __builtin_shufflevector(pop[1], pop[1], 0, 1, 2, 3);
        keep(p0);
        keep(p1);
    }
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

}  // namespace

__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a, const uint8_t* __restrict__ ws) {
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
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // 0..7
    const int team = w >> 2;
    const int wq = w & 3;                                     // query group of this wave
    const int lane = tid & 63;

    // Separate arrays per slot: with the slot parity a compile-time constant
    // in each phase, the compiler can see that the tile being fetched and the
    // tiles being read never overlap, and does not wait for the fetch before
    // reading operands.
    __shared__ __align__(16) uint8_t kslot0[kKSlot];
    __shared__ __align__(16) uint8_t kslot1[kKSlot];
    __shared__ __align__(16) uint8_t vslot0[kVSlot];
    __shared__ __align__(16) uint8_t vslot1[kVSlot];
    __shared__ __align__(16) uint8_t qlds[kQBytes];
    __shared__ __align__(16) int32_t tlist[kListBytes / 4];

    const uint64_t qtile = (uint64_t)bh * nb + qb;
    const int n_tiles = g.n_hi + g.n_lo;

    // The query block's Q operands go first: the E4M3 codes into registers
    // (two 16-byte chunks a thread, widened to bf16 once the tile list below
    // has been gathered) and the E2M1 codes and scales by DMA into LDS.
    uint4 q8c[2];
    {
        const uint8_t* q8_src = ws + a.L.q8 + qtile * (DA2_TILE * DA2_DPAD);
#pragma unroll
        for (int k = 0; k < 2; ++k) q8c[k] = *reinterpret_cast<const uint4*>(q8_src + (tid + kThreads * k) * 16);
        const uint8_t* q4_src = ws + a.L.q4 + qtile * (DA2_TILE * DA2_DPAD / 2);
#pragma unroll
        for (int n = 0; n < 8 / kWaves; ++n) {      // 8 KiB: 8 rows
            const int wr = w + kWaves * n;
            const int p = wr * 64 + lane;
            const int q = p >> 2, pc = p & 3;
            dma16(q4_src + (q * 4 + (pc ^ ((q >> 2) & 3))) * 16, qlds + kQ4 + wr * 1024);
        }
        if (w == 2 && lane < 32)
            dma16(ws + a.L.sq4 + qtile * (DA2_TILE * DA2_DPAD / 32) + lane * 16, qlds + kQs);
    }

    // This query block's tile list, packed with the fp8 exponents, into LDS.
    // The head's K and V exponent rows are staged in the value slots first
    // (coalesced loads), so that no list entry waits for a second global load.
    int32_t* tl = tlist;
    {
        const uint64_t plane = (uint64_t)g.bh * nb;
        uint8_t* ek_row = vslot0;
        uint8_t* ev_row = vslot1;
        for (int i = tid; i < nb; i += kThreads) {
            ek_row[i] = ws[a.L.e8 + plane + (uint64_t)bh * nb + i];
            ev_row[i] = ws[a.L.e8 + 2 * plane + (uint64_t)bh * nb + i];
        }
        const int32_t* hl = reinterpret_cast<const int32_t*>(ws + a.L.hi) + qtile * g.n_hi;
        const int32_t* ll = reinterpret_cast<const int32_t*>(ws + a.L.lo) + qtile * g.n_lo;
        int32_t mine[DA2_MAX_BLOCKS / kThreads];
#pragma unroll
        for (int k = 0; k < DA2_MAX_BLOCKS / kThreads; ++k) {
            const int i = tid + k * kThreads;
            mine[k] = i < g.n_hi ? hl[i] : (i < n_tiles ? ll[i - g.n_hi] : 0);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < DA2_MAX_BLOCKS / kThreads; ++k) {
            const int i = tid + k * kThreads;
            if (i < n_tiles) {
                uint32_t e = (uint32_t)mine[k];
                if (i < g.n_hi) e |= ((uint32_t)ek_row[e] << 16) | ((uint32_t)ev_row[e] << 24);
                tl[i] = (int32_t)e;
            }
        }
    }
    // Q as bf16 (exact widening of the E4M3 codes, without the block scale):
    // 16-byte chunk c (8 channels) of query slot q at chunk c ^ (q & 15)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int ci = tid + kThreads * k;          // 16 codes: slot ci / 8, channels 16 (ci % 8) ..
        const int q = ci >> 3, c = 2 * (ci & 7);
        uint8_t* row = qlds + kQb + q * 256;
        *reinterpret_cast<v8bf*>(row + ((c ^ (q & 15)) << 4)) = widen_e4m3(q8c[k].x, q8c[k].y);
        *reinterpret_cast<v8bf*>(row + (((c + 1) ^ (q & 15)) << 4)) = widen_e4m3(q8c[k].z, q8c[k].w);
    }
    __syncthreads();
    // The first fp8 section's first K tile is fetched now, under the rest of
    // the prologue (team 1 fetches in the even phases).
    if (g.n_hi > 0 && team == 1) {
        const int ln = fresh_lane();
        dma_k<kHi>(tile_from<kHi>(a, ws, bh, tl[0]), kslot0, wq, ln, dma_offsets(ln));
    }
    // Value slot 0 starts zeroed, so that every byte in it is a finite code
    // or scale: the first phase's PV of a section (the empty tile, P = 0)
    // reads it before any fetch has written it. Every other slot is written
    // by a fetch before it is read; in an MXFP4 section slot 0 holds fp8
    // codes (finite in either format) and, in its scale area, which fp8
    // tiles leave untouched, these zeros.
    {
        const uint4 z = {0u, 0u, 0u, 0u};
        for (int i = tid; i < kVSlot / 16; i += kThreads) reinterpret_cast<uint4*>(vslot0)[i] = z;
    }

    WaveState st;
    st.q = qlds;
    st.qs0 = 32 * wq;
    st.m = -__builtin_huge_valf();
    st.mref = -__builtin_huge_valf();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        st.lsum[e] = 0.f;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) st.acc[cb][e] = 0.f;
    }
    // uniform values, kept in scalar registers
    st.c_lo = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, fmaxf((float)g.tau * kLog2E, __FLT_MIN__))));
    st.e_q = __builtin_amdgcn_readfirstlane((int)ws[a.L.e8 + qtile]) - 127;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    v16f s[4];
    v8i pop[2];
    int psc[2];

    // The tile list is run as two sections, its hi tiles and then its lo
    // tiles, each through the same software pipeline; inside a section every
    // step has one precision, so the loop bodies carry no precision branches.
    //
    // Within a section of n tiles, phase p (0 <= p < n + 2): team p%2 runs
    // PV(p-2) and QK^T(p); the other team runs the softmax of tile p-1. So
    // each team owns every other tile: its QK^T in phase j, softmax in phase
    // j+1, PV in phase j+2. K(p+1) and V(p-1) are fetched during phase p into
    // the slots of K(p-1) and V(p-3), whose readers finished in phase p-1;
    // each is waited for at the end of phase p and first read in phase p+1.
    // Each team runs its own copy of the loop, two phases per trip, so the
    // lifetimes of S and P are static and the slot parity of every access is
    // a compile-time constant.
    auto sync = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    // The empty key tile: codes of the section's first tile, bias row
    // n_blocks (all -inf). Its scores are -inf, so its softmax leaves the
    // running max and the accumulator untouched and its P codes are zero,
    // which makes its PV a no-op: the phases before and after a section's
    // tiles run the same code as the others, on it.
    const float* empty_bias = reinterpret_cast<const float*>(ws + a.L.bias) + (uint64_t)nb * DA2_TILE;
    auto section = [&](auto ph, int base, int n) __attribute__((always_inline)) {
        constexpr int PH = decltype(ph)::value;
        // Packed list entry of tile j of this section. The index wraps inside
        // the list array; an entry outside the section is never used.
        auto entry = [&](int j) __attribute__((always_inline)) { return tl[(base + j) & (DA2_MAX_BLOCKS - 1)]; };
        const int32_t e_first = __builtin_amdgcn_readfirstlane(entry(0));
        auto real = [&](int j) __attribute__((always_inline)) { return j >= 0 && j < n; };
        // tile j of the section, or the empty tile
        auto tile = [&](int j, int32_t e) __attribute__((always_inline)) {
            Tile t = tile_from<PH>(a, ws, bh, real(j) ? e : e_first);
            if (!real(j)) {
                t.bias = empty_bias;
                t.e_k = 0;
                t.e_v = 0;
            }
            return t;
        };
        // phase p of the matrix team: PV(p-2) and QK^T(p); ev: entry of tile p-2
        auto mma_phase = [&](auto par, int p, int32_t ev) __attribute__((always_inline)) {
            constexpr int PAR = decltype(par)::value;
            // In fp8 phases the matrix work is the longer: when both waves of
            // a SIMD can issue, this one goes first (in MXFP4 phases the
            // softmax wave does; either other choice measured slower).
            if constexpr (PH == kHi) __builtin_amdgcn_s_setprio(2);
            // the lane coordinates are recomputed here, not kept live
            const int ln = fresh_lane();
            const int q = ln & 31, h = ln >> 5;
            // Q operands for this phase's QK^T are read first, under the PV
            QOps qo;
            load_q<PH>(st, qo, q, h);
            pv<PH>(st, PAR ? vslot1 : vslot0, pop, psc, tile(p - 2, ev).e_v, q, h);
            qk<PH>(PAR ? kslot1 : kslot0, qo, s, q, h);
            if constexpr (PH == kHi) __builtin_amdgcn_s_setprio(0);
        };
        // phase p of the other team: the softmax of tile p-1 (entry ek), with
        // the phase's fetch (fk, fv: entries of K(p+1) and V(p-1)) issued from
        // inside it; K(p+1) and V(p-1) both go to the slots of parity PAR ^ 1.
        auto softmax_phase = [&](auto par, int p, int32_t ek, int32_t fk, int32_t fv) __attribute__((always_inline)) {
            constexpr int PAR = decltype(par)::value;
            // lane offsets recomputed here (a handful of ALU ops) rather than
            // kept live across the loop, where they would be spilled
            const int ln = fresh_lane();
            const DmaOffsets o = dma_offsets(ln);
            const Tile tk = tile(p + 1, fk);
            const Tile tv = tile(p - 1, fv);
            uint8_t* ks = PAR ? kslot0 : kslot1;
            uint8_t* vs = PAR ? vslot0 : vslot1;
            auto fetch = [&]() __attribute__((always_inline)) {
                static_for<kFetchItems<PH>>([&](auto item) __attribute__((always_inline)) {
                    fetch_item<PH, decltype(item)::value>(tk, ks, tv, vs, wq, ln, o);
                    fence();
                });
            };
            // in MXFP4 phases the softmax is the longer work: it issues first
            if constexpr (PH == kLo) __builtin_amdgcn_s_setprio(2);
            softmax<PH>(st, s, tile(p - 1, ek).e_k, pop, psc, fetch);
            if constexpr (PH == kLo) __builtin_amdgcn_s_setprio(0);
        };
        // a list entry read from LDS at the start of a phase becomes a scalar
        // at its end, after the phase's work has hidden the LDS latency
        auto uniform = [&](int32_t v) __attribute__((always_inline)) {
            fence();
            return (int32_t)__builtin_amdgcn_readfirstlane(v);
        };
        using Even = std::integral_constant<int, 0>;
        using Odd = std::integral_constant<int, 1>;
        // the section's first K tile (team 1, which fetches in the even
        // phases; the fp8 section's was issued in the prologue)
        if (PH == kLo && team == 1) {
            const int ln = fresh_lane();
            dma_k<PH>(tile(0, e_first), kslot0, wq, ln, dma_offsets(ln));
        }
        // before the section: the scores of the empty tile, no P
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            psc[n] = 127;
#pragma unroll
            for (int w = 0; w < 8; ++w) pop[n][w] = 0;
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) s[kb][e] = -__builtin_huge_valf();
        // Each team owns the tiles j of its parity and carries three list
        // entries in scalar registers: e_prev (tile j-2, whose PV runs in
        // phase j), e_cur (tile j: softmax and V fetch in phase j+1) and
        // e_next (tile j+2: K fetch in phase j+1). The entry of tile j+4 is
        // read during phase j+1.
        int32_t e_prev = 0;
        int32_t e_cur = __builtin_amdgcn_readfirstlane(entry(team == 0 ? 0 : -1));
        int32_t e_next = __builtin_amdgcn_readfirstlane(entry(team == 0 ? 2 : 1));
        sync();
        // n + 2 phases, rounded up to an even count so that every trip of
        // either team's loop runs one phase of each kind
        const int n_phases = (n + 3) & ~1;
        if (team == 0) {
            for (int p = 0; p < n_phases; p += 2) {
                // tile j = p: e_prev = E[p-2], e_cur = E[p], e_next = E[p+2]
                mma_phase(Even{}, p, e_prev);
                sync();
                const int32_t ahead = entry(p + 4);
                softmax_phase(Odd{}, p + 1, e_cur, e_next, e_cur);
                const int32_t e_new = uniform(ahead);
                sync();
                e_prev = e_cur;
                e_cur = e_next;
                e_next = e_new;
            }
        } else {
            for (int p = 0; p < n_phases; p += 2) {
                // tile j = p - 1: e_cur = E[p-1], e_next = E[p+1]
                const int32_t ahead = entry(p + 3);
                softmax_phase(Even{}, p, e_cur, e_next, e_cur);
                const int32_t e_new = uniform(ahead);
                sync();
                e_prev = e_cur;
                e_cur = e_next;
                e_next = e_new;
                mma_phase(Odd{}, p + 1, e_prev);
                sync();
            }
        }
    };
    if (g.n_hi > 0) section(std::integral_constant<int, kHi>{}, 0, g.n_hi);
    if (g.n_lo > 0) section(std::integral_constant<int, kLo>{}, g.n_hi, g.n_lo);

    const int lq = lane & 31, lh = lane >> 5;
    // ---- merge the two teams: team 1 hands (m, l, acc) to team 0 through LDS ----
    // 65 floats per lane (acc and l): 16640 B per wave, two waves per K slot
    float* xch = reinterpret_cast<float*>(wq < 2 ? kslot0 : kslot1) + (size_t)(wq & 1) * (65 * 64);
    if (team == 1) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) xch[(cb * 16 + e) * 64 + lane] = st.acc[cb][e];
        xch[64 * 64 + lane] = st.lsum[0];
    }
    float* xm = reinterpret_cast<float*>(vslot0) + wq * 64;      // mref: 64 floats per wave
    if (team == 1) xm[lane] = st.mref;
    __syncthreads();
    if (team == 1) return;

    const BlockPos qp = block_pos(g, qb);
    const int b = bh / g.heads;
    const int h = bh - b * g.heads;
    {
        const float m1 = xm[lane];
        const float l1 = xch[64 * 64 + lane];
        const float mm = fmaxf(st.mref, m1);
        const float f0 = st.mref > -__builtin_huge_valf() ? exp2f(st.mref - mm) : 0.0f;
        const float f1 = m1 > -__builtin_huge_valf() ? exp2f(m1 - mm) : 0.0f;
        const float inv = 1.0f / (st.lsum[0] * f0 + l1 * f1);
        const int qs = 32 * wq + lq;
        const int64_t n = slot_raster(g, qp, qs);
        if (n >= 0) {
            const int64_t rowoff = (int64_t)b * g.ostride_b + (int64_t)h * g.ostride_h + n * g.ostride_n;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
                for (int jg = 0; jg < 4; ++jg) {
                    const int c = 32 * cb + 8 * jg + 4 * lh;      // channels c .. c + 3
                    if (c >= g.head_dim) continue;
                    float o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[e] = (st.acc[cb][4 * jg + e] * f0 + xch[(cb * 16 + 4 * jg + e) * 64 + lane] * f1) * inv;
                    if (a.out_fp32) {
                        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + rowoff + c) =
                            make_float4(o[0], o[1], o[2], o[3]);
                    } else {
                        uint2 pk;
                        pk.x = f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16);
                        pk.y = f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16);
                        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + rowoff + c) = pk;
                    }
                }
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
    return launch_kernel(attn_kernel, dim3(total), dim3(kThreads), 0, stream, a, a.ws);
}

}  // namespace da2
