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
//                         64x64 output tile per workgroup, 4x4 per thread.
//   rank_kernel         : per (bh, query block i): row softmax of both maps,
//                         C = (A_avg + A_max) / 2, bitonic sort on
//                         (C descending, index ascending), labels, and the
//                         hi/lo index lists in that rank order.
//   set_labels_kernel   : test hook; ascending lists from given labels by
//                         ballot compaction, count check.
#include "common.hpp"

namespace da2 {

namespace {

constexpr int kTile = 64;
constexpr int kKc = 32;

__global__ __launch_bounds__(256) void draft_logits_kernel(Geo g, const double* __restrict__ pool,
                                                           double* __restrict__ logits) {
    const int m = blockIdx.z & 1;           // 0 = avg map, 1 = max map
    const int bh = blockIdx.z >> 1;
    const int i0 = blockIdx.y * kTile;
    const int j0 = blockIdx.x * kTile;
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int nb = g.n_blocks;
    const uint64_t plane = (uint64_t)g.bh * nb * DA2_DPAD;
    const double* qp = pool + (uint64_t)(m) * plane + (uint64_t)bh * nb * DA2_DPAD;       // q avg / q max
    const double* kp = pool + (uint64_t)(2 + m) * plane + (uint64_t)bh * nb * DA2_DPAD;   // k avg / k max

    __shared__ double qs[kTile][kKc + 1];
    __shared__ double ks[kTile][kKc + 1];
    double acc[4][4] = {};
    for (int c0 = 0; c0 < g.head_dim; c0 += kKc) {
        for (int e = tid; e < kTile * kKc; e += 256) {
            const int r = e / kKc, cc = e % kKc;
            qs[r][cc] = (i0 + r < nb) ? qp[(uint64_t)(i0 + r) * DA2_DPAD + c0 + cc] : 0.0;
            ks[r][cc] = (j0 + r < nb) ? kp[(uint64_t)(j0 + r) * DA2_DPAD + c0 + cc] : 0.0;
        }
        __syncthreads();
#pragma unroll 4
        for (int cc = 0; cc < kKc; ++cc) {
            double qa[4], kb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                qa[u] = qs[ty + 16 * u][cc];
                kb[u] = ks[tx + 16 * u][cc];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int w = 0; w < 4; ++w) acc[u][w] = fma(qa[u], kb[w], acc[u][w]);
        }
        __syncthreads();
    }
    double* out = logits + (uint64_t)m * g.bh * nb * nb + (uint64_t)bh * nb * nb;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int i = i0 + ty + 16 * u, j = j0 + tx + 16 * w;
            if (i < nb && j < nb) out[(uint64_t)i * nb + j] = g.tau * acc[u][w];
        }
}

__device__ __forceinline__ double block_reduce_max(double v, double* red) {
    for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
}

__device__ __forceinline__ double block_reduce_sum(double v, double* red) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
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
    return count;
}

__global__ __launch_bounds__(256) void rank_kernel(Geo g, double* __restrict__ scores, int8_t* __restrict__ labels,
                                                   int32_t* __restrict__ hi_list, int32_t* __restrict__ lo_list) {
    const int i = blockIdx.x;
    const int bh = blockIdx.y;
    const int nb = g.n_blocks;
    const int tid = threadIdx.x;
    int np = 1;
    while (np < nb) np <<= 1;

    extern __shared__ __align__(16) unsigned char smem[];
    double* val = reinterpret_cast<double*>(smem);              // [np]
    int32_t* idx = reinterpret_cast<int32_t*>(val + np);        // [np]
    int8_t* lab = reinterpret_cast<int8_t*>(idx + np);          // [np]
    __shared__ double red[4];

    double* row_avg = scores + ((uint64_t)bh * nb + i) * nb;
    double* row_max = scores + (uint64_t)g.bh * nb * nb + ((uint64_t)bh * nb + i) * nb;

    // combined score C = (softmax(avg row) + softmax(max row)) / 2
    double mx = -__builtin_huge_val();
    for (int j = tid; j < nb; j += 256) mx = fmax(mx, row_avg[j]);
    mx = block_reduce_max(mx, red);
    double sm = 0.0;
    for (int j = tid; j < nb; j += 256) {
        const double e = exp(row_avg[j] - mx);
        val[j] = e;
        sm += e;
    }
    sm = block_reduce_sum(sm, red);
    double mx2 = -__builtin_huge_val();
    for (int j = tid; j < nb; j += 256) mx2 = fmax(mx2, row_max[j]);
    mx2 = block_reduce_max(mx2, red);
    double sm2 = 0.0;
    for (int j = tid; j < nb; j += 256) sm2 += exp(row_max[j] - mx2);
    sm2 = block_reduce_sum(sm2, red);
    for (int j = tid; j < np; j += 256) {
        if (j < nb) {
            const double c = 0.5 * (val[j] / sm + exp(row_max[j] - mx2) / sm2);
            val[j] = c;
            idx[j] = j;
            row_avg[j] = c;     // section 0 of the scores now holds C for this row
        } else {
            val[j] = -1.0;      // sorts after every real score (C >= 0)
            idx[j] = j;
        }
    }
    __syncthreads();

    // bitonic sort, "a before b" iff C_a > C_b or (C_a == C_b and index_a < index_b).
    // Thread tid owns the compare pairs p = tid, tid + 256, ...; for a partner
    // distance jj <= 64 the pairs of wave w touch only elements 128 w ..
    // 128 w + 127 (and the same plus multiples of 512), so consecutive such
    // steps need no workgroup barrier (a wave's LDS accesses complete in order).
    for (int k = 2; k <= np; k <<= 1) {
        for (int jj = k >> 1; jj > 0; jj >>= 1) {
            const int lg = __builtin_ctz(jj);
            for (int p = tid; p < (np >> 1); p += 256) {
                const int lo = ((p >> lg) << (lg + 1)) + (p & (jj - 1));
                const int hi = lo + jj;
                const double va = val[lo], vb = val[hi];
                const int ia = idx[lo], ib = idx[hi];
                const bool b_first = (vb > va) || (vb == va && ib < ia);
                const bool a_first = (va > vb) || (va == vb && ia < ib);
                const bool forward = (lo & k) == 0;
                if (forward ? b_first : a_first) {
                    val[lo] = vb;
                    val[hi] = va;
                    idx[lo] = ib;
                    idx[hi] = ia;
                }
            }
            // A workgroup barrier is needed when this step or the next one
            // crosses waves (distance above 64); the next step's distance is
            // jj / 2, or k when this stage ends. (With np > 512 a thread's
            // second pair p + 256 lies 512 elements further, in the same
            // wave's other chunk, which keeps small distances wave-local.)
            if (jj > 64 || (jj == 1 && k > 64))
                __syncthreads();
            else
                __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();
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
    hipError_t e = launch_kernel(draft_logits_kernel, dim3(t, t, 2 * g.bh), dim3(256), 0, stream, g, pool, scores);
    if (e != hipSuccess) return e;
    int np = 1;
    while (np < g.n_blocks) np <<= 1;
    const size_t shmem = (size_t)np * (8 + 4 + 1);
    return launch_kernel(rank_kernel, dim3(g.n_blocks, g.bh), dim3(256), shmem, stream, g, scores,
                       reinterpret_cast<int8_t*>(base + L.labels), reinterpret_cast<int32_t*>(base + L.hi),
                       reinterpret_cast<int32_t*>(base + L.lo));
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
