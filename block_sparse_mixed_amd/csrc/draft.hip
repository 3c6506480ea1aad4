// K2: draft attention map and the shared ranking.
//
// [DraftAttention2 (arXiv 2609.32628), abstract]: average- and max-pooled
// queries and keys estimate block importance through a low-resolution draft
// attention map; one shared ranking per query block gives the top blocks the
// higher precision, the next retained blocks the lower precision, and skips
// the rest under configurable budgets. [DraftAttention (arXiv 2505.14708),
// abstract]: the draft map is attention between the down-sampled queries and
// keys across all frames.
//
// Scores are computed in fp64 so that the ranking agrees with a float64
// reference except for genuine near-ties: fp32 dot products of 128 pooled
// channels carry ~1e-5 relative error, which is larger than the 1e-5 band in
// which either adjacent label is accepted.
//
//   draft_logits_kernel : L[m][bh][i][j] = tau * <P_m,q[i], P_m,k[j]>, m in {avg, max};
//                         32x32 output tile per workgroup, fp64 MFMAs.
//   rank_wave_kernel    : per (bh, query block i), one wave (rows of up to
//   rank_kernel           1024 blocks) or one workgroup (larger rows): row
//                         softmax of both maps, C = (A_avg + A_max) / 2,
//                         bitonic sort on (C descending, index ascending),
//                         labels, and the hi/lo index lists in that rank order.
//   set_labels_kernel   : test hook; ascending lists from given labels by
//                         ballot compaction, count check.
#include "common.hpp"

namespace da2 {

namespace {

constexpr int kTile = 32;

typedef double v4d __attribute__((ext_vector_type(4)));

// One workgroup: a 32 x 32 tile of one map's logits, as 2 x 2 fp64 MFMA
// tiles (V_MFMA_F64_16X16X4_F64: lane l gives A row l % 16 and B column
// l % 16 at k = l / 16, and gets D rows l / 16 + 4 e, e = 0 .. 3, of column
// l % 16). The four waves split the channels, 32 each, so that every wave
// issues all of its loads at once and the memory latency is paid once per
// workgroup rather than once per channel chunk; their partial sums then add
// up through LDS in a fixed order. Within a wave the channel order of the
// contraction is free as long as both operands agree: lane group
// g = l / 16 feeds channels 32 w + 8 g + s to the step-s MFMA, so that
// every lane reads 64 contiguous bytes of each of its rows. The sums run in
// fp64, each product and addition rounded once, as in a plain loop of fused
// multiply-adds (in another order).
// A one-dimensional grid of (map, head) slices times t x t tiles, in an
// XCD-aware order: the workgroups one XCD receives (every eighth) take
// consecutive tiles of the same slices, so that a slice's pooled rows are
// fetched into one L2 rather than into all eight.
__global__ __launch_bounds__(256) void draft_logits_kernel(Geo g, const double* __restrict__ pool,
                                                           double* __restrict__ logits) {
    const int nb = g.n_blocks;
    const int t = (nb + kTile - 1) / kTile;
    const int total = 2 * g.bh * t * t;
    const int xcd = blockIdx.x & 7, k8 = blockIdx.x >> 3;
    const int per = total >> 3, rem = total & 7;
    const int logical = xcd * per + min(xcd, rem) + k8;
    const int slice = logical / (t * t), tile = logical - slice * (t * t);
    const int m = slice & 1;                // 0 = avg map, 1 = max map
    const int bh = slice >> 1;
    const int i0 = (tile / t) * kTile, j0 = (tile % t) * kTile;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t plane = (uint64_t)g.bh * nb * DA2_DPAD;
    const double* qp = pool + (uint64_t)(m) * plane + (uint64_t)bh * nb * DA2_DPAD;       // q avg / q max
    const double* kp = pool + (uint64_t)(2 + m) * plane + (uint64_t)bh * nb * DA2_DPAD;   // k avg / k max
    const int r = lane & 15, kg = lane >> 4;
    const int c0 = 32 * w + 8 * kg;         // this lane's first channel
    const bool chan = 32 * w < g.head_dim;  // the wave has channels to sum

    v4d acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = (v4d){0.0, 0.0, 0.0, 0.0};
    if (chan) {
        // A rows (queries) i0 + 16 tt + r, B rows (keys) j0 + 16 tt + r; a
        // row past the end is read from row 0, unconditionally, and zeroed
        double ca[2][8], cb[2][8];
        auto load = [&](double (&x)[8], const double* base, int row) __attribute__((always_inline)) {
            const bool ok = row < nb;
            const double2* src = reinterpret_cast<const double2*>(base + (uint64_t)(ok ? row : 0) * DA2_DPAD + c0);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const double2 v = src[u];
                x[2 * u] = ok ? v.x : 0.0;
                x[2 * u + 1] = ok ? v.y : 0.0;
            }
        };
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            load(ca[tt], qp, i0 + 16 * tt + r);
            load(cb[tt], kp, j0 + 16 * tt + r);
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(ca[0][s], cb[0][s], acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(ca[0][s], cb[1][s], acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(ca[1][s], cb[0][s], acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(ca[1][s], cb[1][s], acc[1][1], 0, 0, 0);
        }
    }
    // partial sums [wave][MFMA tile][element][lane], then each thread adds the
    // four waves' values of four outputs in wave order
    __shared__ double part[4][4][4][64];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) part[w][k][e][lane] = acc[k >> 1][k & 1][e];
    __syncthreads();
    double* out = logits + (uint64_t)m * g.bh * nb * nb + (uint64_t)bh * nb * nb;
    const int e = w;                        // this thread's element index
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const double v = ((part[0][k][e][lane] + part[1][k][e][lane]) + part[2][k][e][lane]) + part[3][k][e][lane];
        const int i = i0 + 16 * (k >> 1) + kg + 4 * e, j = j0 + 16 * (k & 1) + r;
        if (i < nb && j < nb) out[(uint64_t)i * nb + j] = g.tau * v;
    }
}

// The value of lane l ^ D (D < 64, a power of two) without a trip through
// LDS for most D: quad permutes for 1 and 2, a row rotation for 8 (rows of
// 16 lanes), the 16- and 32-lane swaps for 16 and 32, and a swizzle for 4.
template <int D>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
    const int lane = threadIdx.x & 63;
    if constexpr (D == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
    } else if constexpr (D == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
    } else if constexpr (D == 4) {
        return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, (4 << 10) | 0x1F);      // xor 4 within 32 lanes
    } else if constexpr (D == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false);   // row_ror:8
    } else if constexpr (D == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane & 16) ? r[0] : r[1];
    } else {
        static_assert(D == 32, "lane distance");
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane & 32) ? r[0] : r[1];
    }
}
template <int D>
__device__ __forceinline__ double lane_xor(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = lane_xor<D>((uint32_t)u), hi = lane_xor<D>((uint32_t)(u >> 32));
    return __builtin_bit_cast(double, lo | (hi << 32));
}

// Workgroup (four waves) maximum and sum of two values at once; each value
// is reduced exactly as a reduction of its own would (butterfly within the
// wave, then the four wave results in a fixed order).
template <int D>
__device__ __forceinline__ void butterfly_max2(double& a, double& b) {
    a = fmax(a, lane_xor<D>(a));
    b = fmax(b, lane_xor<D>(b));
    if constexpr (D > 1) butterfly_max2<D / 2>(a, b);
}
template <int D>
__device__ __forceinline__ void butterfly_sum2(double& a, double& b) {
    a += lane_xor<D>(a);
    b += lane_xor<D>(b);
    if constexpr (D > 1) butterfly_sum2<D / 2>(a, b);
}

__device__ __forceinline__ void block_reduce_max2(double& a, double& b, double* red) {
    butterfly_max2<32>(a, b);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        red[w] = a;
        red[4 + w] = b;
    }
    __syncthreads();
    a = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
    b = fmax(fmax(red[4], red[5]), fmax(red[6], red[7]));
}

__device__ __forceinline__ void block_reduce_sum2(double& a, double& b, double* red) {
    butterfly_sum2<32>(a, b);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        red[w] = a;
        red[4 + w] = b;
    }
    __syncthreads();
    a = (red[0] + red[1]) + (red[2] + red[3]);
    b = (red[4] + red[5]) + (red[6] + red[7]);
}

// Write the ascending lists of blocks labelled want (at most cap entries);
// executed by one wave. Returns the number found.
__device__ __forceinline__ int compact_list(const int8_t* lab, int nb, int8_t want, int32_t* out, int cap) {
    const int lane = threadIdx.x & 63;
    int count = 0;
    for (int j0 = 0; j0 < nb; j0 += 64) {
        const int j = j0 + lane;
        const bool hit = j < nb && lab[j] == want;
        const unsigned long long mask = __ballot(hit);
        const int p = count + __popcll(mask & ((1ull << lane) - 1ull));
        if (hit && p < cap) out[p] = j;
        count += __popcll(mask);
    }
    // a row with fewer such labels than the list holds: the rest of the list
    // gets block 0, so that every list entry names a real block
    for (int p = count + lane; p < cap; p += 64) out[p] = 0;
    return count;
}

// The value a block's score C sorts by: C itself (C >= 0), or -0.5 for a NaN
// score (non-finite inputs), so that the order stays total, such blocks rank
// after every real score and before the padding (-1.0), and the lists remain
// a permutation of real blocks whatever the inputs held.
__device__ __forceinline__ double sort_key(double c) { return c >= 0.0 ? c : -0.5; }

// "a before b" in rank order: larger C first, then the lower block index.
// Bitwise operators, so that the three comparisons combine as lane masks
// rather than as branches.
__device__ __forceinline__ bool before(double va, int ia, double vb, int ib) {
    return (va > vb) | ((va == vb) & (ia < ib));
}

// Bitonic sort of np = 256 R (value, index) pairs held in registers: lane l
// of wave w holds elements 64 R w + R l .. + R - 1. A compare-exchange step
// of partner distance jj runs inside the lane (jj < R), across lanes of the
// wave by shuffles (jj < 64 R), or across waves through LDS (the only steps
// with workgroup barriers). The pairs start in and return to val/idx.
template <int R>
struct SortState {
    double v[R];
    int ix[R];
};

// One compare-exchange step of stage k, partner distance jj: element e ends
// up holding the first of the pair (e, e ^ jj) when it is the lower element
// of an ascending pair or the upper element of a descending one.
// D: the lane distance jj / R when it is known at compile time (0 otherwise)
// In-lane compare-exchange at a compile-time distance J < R, so that every
// register index is a constant (a run-time distance would index the arrays
// dynamically and move them to scratch memory).
template <int R, int J>
__device__ __forceinline__ void inlane_step(SortState<R>& st, int base, int k) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r & J) continue;
        const int r2 = r | J;
        const bool fwd = ((base + r) & k) == 0;
        const bool swap = fwd != before(st.v[r], st.ix[r], st.v[r2], st.ix[r2]);
        const double a = st.v[r], b = st.v[r2];
        const int ia = st.ix[r], ib = st.ix[r2];
        st.v[r] = swap ? b : a;
        st.v[r2] = swap ? a : b;
        st.ix[r] = swap ? ib : ia;
        st.ix[r2] = swap ? ia : ib;
    }
}

// run-time distance jj < R -> the matching compile-time step
template <int R, int J = 1>
__device__ __forceinline__ void inlane_dispatch(SortState<R>& st, int base, int k, int jj) {
    if constexpr (J < R) {
        if (jj == J) {
            inlane_step<R, J>(st, base, k);
            return;
        }
        inlane_dispatch<R, 2 * J>(st, base, k, jj);
    }
}

template <int R, int D = 0>
__device__ __forceinline__ void bitonic_step(SortState<R>& st, double* val, int32_t* idx, int base, int k, int jj) {
    if (jj < R) {
        inlane_dispatch<R>(st, base, k, jj);
        return;
    }
    double pv[R];
    int pi[R];
    if (jj < 64 * R) {
        const int d = jj / R;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if constexpr (D > 0) {
                pv[r] = lane_xor<D>(st.v[r]);
                pi[r] = (int)lane_xor<D>((uint32_t)st.ix[r]);
            } else {
                pv[r] = __shfl_xor(st.v[r], d);
                pi[r] = __shfl_xor(st.ix[r], d);
            }
        }
    } else {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            val[base + r] = st.v[r];
            idx[base + r] = st.ix[r];
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            pv[r] = val[(base + r) ^ jj];
            pi[r] = idx[(base + r) ^ jj];
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e = base + r;
        const bool want_first = ((e & jj) == 0) == ((e & k) == 0);
        const bool take = before(st.v[r], st.ix[r], pv[r], pi[r]) != want_first;
        st.v[r] = take ? pv[r] : st.v[r];
        st.ix[r] = take ? pi[r] : st.ix[r];
    }
}

// Every stage and step at compile time, so that every condition of a step
// folds away and the pairs stay in registers. A run-time loop over the
// steps (tried for rows of 2048 and 4096 pairs) made the compiler keep the
// pairs in scratch memory and ranked 4.4-5.3 times slower.
template <int R, int K, int JJ, int NP = 256 * R>
__device__ __forceinline__ void bitonic_stages(SortState<R>& st, double* val, int32_t* idx, int base) {
    if constexpr (K <= NP) {
        bitonic_step<R, (JJ >= R && JJ < 64 * R) ? JJ / R : 0>(st, val, idx, base, K, JJ);
        if constexpr (JJ > 1)
            bitonic_stages<R, K, JJ / 2, NP>(st, val, idx, base);
        else
            bitonic_stages<R, 2 * K, K, NP>(st, val, idx, base);
    }
}

// Bitonic sort of np = 256 R (value, index) pairs held in registers: lane l
// of wave w holds elements 64 R w + R l .. + R - 1. A compare-exchange step
// of partner distance jj runs inside the lane (jj < R), across lanes of the
// wave by shuffles (jj < 64 R), or across waves through LDS (the only steps
// with workgroup barriers). The pairs start in and return to val/idx.
template <int R>
__device__ __forceinline__ void bitonic_sort(double* val, int32_t* idx) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int base = 64 * R * w + R * lane;
    SortState<R> st;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        st.v[r] = val[base + r];
        st.ix[r] = idx[base + r];
    }
    bitonic_stages<R, 2, 1>(st, val, idx, base);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        val[base + r] = st.v[r];
        idx[base + r] = st.ix[r];
    }
    __syncthreads();
}

// R = np / 256 pairs per thread in the sort (a template parameter, so that
// each size gets its own register allocation)
template <int R>
__global__ __launch_bounds__(256) void rank_kernel(Geo g, double* __restrict__ scores, int8_t* __restrict__ labels,
                                                   int32_t* __restrict__ hi_list, int32_t* __restrict__ lo_list) {
    const int i = blockIdx.x;
    const int bh = blockIdx.y;
    const int nb = g.n_blocks;
    const int tid = threadIdx.x;
    const int np = 256 * R;         // a power of two, at least nb and one pair per thread

    extern __shared__ __align__(16) unsigned char smem[];
    double* val = reinterpret_cast<double*>(smem);              // [np]
    double* val2 = val + np;                                    // [np]
    int32_t* idx = reinterpret_cast<int32_t*>(val2 + np);       // [np]
    int8_t* lab = reinterpret_cast<int8_t*>(idx + np);          // [np]
    __shared__ double red[8];

    double* row_avg = scores + ((uint64_t)bh * nb + i) * nb;
    double* row_max = scores + (uint64_t)g.bh * nb * nb + ((uint64_t)bh * nb + i) * nb;

    // combined score C = (softmax(avg row) + softmax(max row)) / 2; both rows
    // are read from global memory once, into LDS
    double mx = -__builtin_huge_val(), mx2 = -__builtin_huge_val();
    for (int j = tid; j < nb; j += 256) {
        const double va = row_avg[j], vm = row_max[j];
        val[j] = va;
        val2[j] = vm;
        mx = fmax(mx, va);
        mx2 = fmax(mx2, vm);
    }
    block_reduce_max2(mx, mx2, red);
    double sm = 0.0, sm2 = 0.0;
    for (int j = tid; j < nb; j += 256) {
        const double e = exp(val[j] - mx), e2 = exp(val2[j] - mx2);
        val[j] = e;
        val2[j] = e2;
        sm += e;
        sm2 += e2;
    }
    block_reduce_sum2(sm, sm2, red);
    for (int j = tid; j < np; j += 256) {
        if (j < nb) {
            const double c = 0.5 * (val[j] / sm + val2[j] / sm2);
            val[j] = sort_key(c);
            idx[j] = j;
            row_avg[j] = c;     // section 0 of the scores now holds C for this row
        } else {
            val[j] = -1.0;      // sorts after every real score (C >= 0)
            idx[j] = j;
        }
    }
    __syncthreads();

    // bitonic sort, "a before b" iff C_a > C_b or (C_a == C_b and index_a < index_b)
    bitonic_sort<R>(val, idx);
    const int n_ret = g.n_hi + g.n_lo;
    for (int r = tid; r < nb; r += 256) lab[idx[r]] = (int8_t)(r < g.n_hi ? DA2_HI : (r < n_ret ? DA2_LO : DA2_SKIP));
    __syncthreads();
    int8_t* lrow = labels + ((uint64_t)bh * nb + i) * nb;
    for (int j = tid; j < nb; j += 256) lrow[j] = lab[j];
    // lists in rank order (best first): the attention kernel then meets each
    // row's largest scores early and rarely has to rescale its accumulator
    const uint64_t rowid = (uint64_t)bh * nb + i;
    for (int r = tid; r < n_ret; r += 256) {
        if (r < g.n_hi)
            hi_list[rowid * g.n_hi + r] = idx[r];
        else
            lo_list[rowid * g.n_lo + (r - g.n_hi)] = idx[r];
    }
}

// The same ranking with one wave per row, for rows of at most 1024 blocks
// (np = 64 R): the row's values stay in the wave's registers from the loads
// through the sort (lane l holds elements R l .. R l + R - 1), so no step
// needs LDS or a barrier; only the labels pass through LDS, to be written
// out in raster order. Four rows per workgroup.
template <int R>
__global__ __launch_bounds__(256) void rank_wave_kernel(Geo g, double* __restrict__ scores, int8_t* __restrict__ labels,
                                                        int32_t* __restrict__ hi_list, int32_t* __restrict__ lo_list) {
    constexpr int np = 64 * R;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int i = blockIdx.x * 4 + w;
    const int bh = blockIdx.y;
    const int nb = g.n_blocks;
    __shared__ int8_t lab_all[4][np];
    if (i >= nb) return;                 // no barriers below
    int8_t* lab = lab_all[w];
    double* row_avg = scores + ((uint64_t)bh * nb + i) * nb;
    const double* row_max = scores + (uint64_t)g.bh * nb * nb + ((uint64_t)bh * nb + i) * nb;
    const int base = R * lane;

    // combined score C = (softmax(avg row) + softmax(max row)) / 2
    double va[R], vm[R];
    double mx = -__builtin_huge_val(), mx2 = -__builtin_huge_val();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int j = base + r;
        va[r] = j < nb ? row_avg[j] : -__builtin_huge_val();
        vm[r] = j < nb ? row_max[j] : -__builtin_huge_val();
        mx = fmax(mx, va[r]);
        mx2 = fmax(mx2, vm[r]);
    }
    butterfly_max2<32>(mx, mx2);
    double sm = 0.0, sm2 = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        va[r] = base + r < nb ? exp(va[r] - mx) : 0.0;
        vm[r] = base + r < nb ? exp(vm[r] - mx2) : 0.0;
        sm += va[r];
        sm2 += vm[r];
    }
    butterfly_sum2<32>(sm, sm2);
    SortState<R> st;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int j = base + r;
        st.ix[r] = j;
        if (j < nb) {
            const double c = 0.5 * (va[r] / sm + vm[r] / sm2);
            st.v[r] = sort_key(c);
            row_avg[j] = c;         // section 0 of the scores now holds C for this row
        } else {
            st.v[r] = -1.0;         // sorts after every real score (C >= 0)
        }
    }

    // bitonic sort, "a before b" iff C_a > C_b or (C_a == C_b and index_a < index_b);
    // every step's partner is in the lane or in the wave
    bitonic_stages<R, 2, 1, np>(st, nullptr, nullptr, base);

    const int n_ret = g.n_hi + g.n_lo;
    const uint64_t rowid = (uint64_t)bh * nb + i;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int pos = base + r;      // rank of the element this lane now holds
        if (pos < nb) lab[st.ix[r]] = (int8_t)(pos < g.n_hi ? DA2_HI : (pos < n_ret ? DA2_LO : DA2_SKIP));
        // lists in rank order (best first)
        if (pos < g.n_hi)
            hi_list[rowid * g.n_hi + pos] = st.ix[r];
        else if (pos < n_ret)
            lo_list[rowid * g.n_lo + (pos - g.n_hi)] = st.ix[r];
    }
    // the wave's own LDS writes, read back by its other lanes: LDS
    // instructions of one wave complete in order; the fence keeps the
    // compiler from moving the reads above the writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int8_t* lrow = labels + rowid * nb;
    for (int j = lane; j < nb; j += 64) lrow[j] = lab[j];
}

__global__ __launch_bounds__(64) void set_labels_kernel(Geo g, const int8_t* __restrict__ src, int8_t* __restrict__ labels,
                                                        int32_t* __restrict__ hi_list, int32_t* __restrict__ lo_list,
                                                        uint32_t* __restrict__ status) {
    const int i = blockIdx.x;
    const int bh = blockIdx.y;
    const int nb = g.n_blocks;
    const uint64_t rowid = (uint64_t)bh * nb + i;
    const int8_t* srow = src + rowid * nb;
    int8_t* drow = labels + rowid * nb;
    for (int j = threadIdx.x; j < nb; j += 64) drow[j] = srow[j];
    const int nh = compact_list(srow, nb, DA2_HI, hi_list + rowid * (g.n_hi > 0 ? g.n_hi : 1), g.n_hi);
    const int nl = compact_list(srow, nb, DA2_LO, lo_list + rowid * (g.n_lo > 0 ? g.n_lo : 1), g.n_lo);
    if (threadIdx.x == 0 && (nh != g.n_hi || nl != g.n_lo)) atomicAdd(status, 1u);
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
    const int i = threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_draft(const Geo& g, const Layout& L, void* ws, hipStream_t stream) {
    uint8_t* base = static_cast<uint8_t*>(ws);
    const double* pool = reinterpret_cast<const double*>(base + L.pool);
    double* scores = reinterpret_cast<double*>(base + L.scores);
    const int t = (g.n_blocks + kTile - 1) / kTile;
    hipError_t e = launch_kernel(draft_logits_kernel, dim3(2 * g.bh * t * t), dim3(256), 0, stream, g, pool, scores);
    if (e != hipSuccess) return e;
    int np = 256;
    while (np < g.n_blocks) np <<= 1;
    if (np <= 1024) {
        auto run_wave = [&](auto kernel) {
            return launch_kernel(kernel, dim3((g.n_blocks + 3) / 4, g.bh), dim3(256), 0, stream, g, scores,
                                 reinterpret_cast<int8_t*>(base + L.labels), reinterpret_cast<int32_t*>(base + L.hi),
                                 reinterpret_cast<int32_t*>(base + L.lo));
        };
        switch (np) {
            case 256: return run_wave(rank_wave_kernel<4>);
            case 512: return run_wave(rank_wave_kernel<8>);
            default: return run_wave(rank_wave_kernel<16>);
        }
    }
    const size_t shmem = (size_t)np * (8 + 8 + 4 + 1);
    auto run = [&](auto kernel) {
        return launch_kernel(kernel, dim3(g.n_blocks, g.bh), dim3(256), shmem, stream, g, scores,
                             reinterpret_cast<int8_t*>(base + L.labels), reinterpret_cast<int32_t*>(base + L.hi),
                             reinterpret_cast<int32_t*>(base + L.lo));
    };
    switch (np >> 8) {
        case 8: return run(rank_kernel<8>);
        default: return run(rank_kernel<16>);      // np <= DA2_MAX_BLOCKS = 4096
    }
}

hipError_t launch_set_labels(const Geo& g, const Layout& L, void* ws, const int8_t* labels, hipStream_t stream) {
    uint8_t* base = static_cast<uint8_t*>(ws);
    uint32_t* status = reinterpret_cast<uint32_t*>(base + L.status);
    hipError_t e = launch_kernel(zero_u32_kernel, dim3(1), dim3(64), 0, stream, status, 4);
    if (e != hipSuccess) return e;
    return launch_kernel(set_labels_kernel, dim3(g.n_blocks, g.bh), dim3(64), 0, stream, g, labels,
                       reinterpret_cast<int8_t*>(base + L.labels), reinterpret_cast<int32_t*>(base + L.hi),
                       reinterpret_cast<int32_t*>(base + L.lo), status);
}

}  // namespace da2
