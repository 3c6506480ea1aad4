// Host-side plan: validation, window geometry, budget counts, workspace layout.
// Built without floating-point contraction so that the budget counts are the
// IEEE-double evaluation of the formulas as written.
#include <cmath>
#include <cstdlib>
#include <new>

#include "da2_internal.hpp"

namespace {

uint64_t align256(uint64_t x) { return (x + 255u) & ~uint64_t(255u); }

}  // namespace

extern "C" da2_status da2_plan(const da2_config* cfg, da2_plan_t** out) {
    if (!cfg || !out) return DA2_ERR_INVALID_ARG;
    *out = nullptr;
    const da2_config& c = *cfg;
    if (c.batch <= 0 || c.heads <= 0 || c.frames <= 0 || c.grid_h <= 0 || c.grid_w <= 0 ||
        c.head_dim <= 0 || c.win_h <= 0 || c.win_w <= 0)
        return DA2_ERR_INVALID_ARG;
    if ((c.flags & ~(uint32_t)DA2_FLAG_PACK_EDGES) != 0) return DA2_ERR_INVALID_ARG;
    if (c.out_dtype != DA2_OUT_BF16 && c.out_dtype != DA2_OUT_FP32) return DA2_ERR_INVALID_ARG;
    if (!(c.budget_hi >= 0.0 && c.budget_hi <= 1.0 && c.budget_lo >= 0.0 && std::isfinite(c.budget_lo)))
        return DA2_ERR_INVALID_ARG;
    if (!(c.softmax_scale >= 0.0) || !std::isfinite(c.softmax_scale)) return DA2_ERR_INVALID_ARG;
    if (c.stride_b < 0 || c.stride_h < 0 || c.stride_n < 0) return DA2_ERR_INVALID_ARG;
    if (c.out_stride_b < 0 || c.out_stride_h < 0 || c.out_stride_n < 0) return DA2_ERR_INVALID_ARG;
    if (c.head_dim % 32 != 0 || c.head_dim > DA2_DPAD) return DA2_ERR_UNSUPPORTED;
    if ((int64_t)c.win_h * c.win_w > DA2_TILE) return DA2_ERR_UNSUPPORTED;

    da2::Geo g{};
    g.frames = c.frames;
    g.grid_h = c.grid_h;
    g.grid_w = c.grid_w;
    g.win_h = c.win_h;
    g.win_w = c.win_w;
    const int64_t n_wy = ((int64_t)c.grid_h + c.win_h - 1) / c.win_h;
    const int64_t n_wx = ((int64_t)c.grid_w + c.win_w - 1) / c.win_w;
    int64_t nb = (int64_t)c.frames * n_wy * n_wx;
    if (nb > DA2_MAX_BLOCKS) return DA2_ERR_UNSUPPORTED;
    g.n_wy = (int32_t)n_wy;
    g.n_wx = (int32_t)n_wx;
    g.block_size = c.win_h * c.win_w;
    g.pack = (c.flags & DA2_FLAG_PACK_EDGES) ? 1 : 0;
    g.fwy = c.grid_h / c.win_h;
    g.fwx = c.grid_w / c.win_w;
    g.n_full = (int32_t)((int64_t)c.frames * g.fwy * g.fwx);
    g.edge_frame = c.grid_h * c.grid_w - g.fwy * g.fwx * g.block_size;
    g.edge_total = (int32_t)((int64_t)c.frames * g.edge_frame);   // < the padded slot count, which fits
    if (g.pack) nb = g.n_full + ((int64_t)g.edge_total + g.block_size - 1) / g.block_size;
    g.n_blocks = (int32_t)nb;
    g.head_dim = c.head_dim;
    g.heads = c.heads;
    int64_t bh = (int64_t)c.batch * c.heads;
    if (bh > 65535) return DA2_ERR_UNSUPPORTED;
    // Every launch's size along x, in work-items, fits the 32 bits of the
    // dispatch: the attention kernel runs one 512-thread workgroup per
    // (b*h, query block), the draft logits one 256-thread workgroup per 32x32
    // tile of each of the two maps of every b*h.
    {
        const uint64_t t = (uint64_t)(nb + 31) / 32;
        if ((uint64_t)bh * (uint64_t)nb * 512u > UINT32_MAX || 2u * (uint64_t)bh * t * t * 256u > UINT32_MAX)
            return DA2_ERR_UNSUPPORTED;
    }
    g.bh = (int32_t)bh;
    g.tokens = (int64_t)c.frames * c.grid_h * c.grid_w;

    // budget counts, evaluated step by step in IEEE double
    double lo_frac = c.budget_lo;
    double hi_rest = 1.0 - c.budget_hi;
    if (lo_frac > hi_rest) lo_frac = hi_rest;
    double nbd = (double)nb;
    double hi_prod = c.budget_hi * nbd;
    double hi_half = hi_prod + 0.5;
    double ret_frac = c.budget_hi + lo_frac;
    double ret_prod = ret_frac * nbd;
    double ret_half = ret_prod + 0.5;
    int64_t n_hi = (int64_t)std::floor(hi_half);
    int64_t n_ret = (int64_t)std::floor(ret_half);
    if (n_ret < 1) return DA2_ERR_INVALID_ARG;
    if (n_ret > nb) n_ret = nb;
    if (n_hi > n_ret) n_hi = n_ret;
    g.n_hi = (int32_t)n_hi;
    g.n_lo = (int32_t)(n_ret - n_hi);

    if (c.stride_b == 0 && c.stride_h == 0 && c.stride_n == 0) {
        g.stride_n = c.head_dim;
        g.stride_h = g.tokens * c.head_dim;
        g.stride_b = c.heads * g.stride_h;
    } else {
        if (c.stride_n < c.head_dim || c.stride_h <= 0 || c.stride_b <= 0) return DA2_ERR_INVALID_ARG;
        g.stride_n = c.stride_n;
        g.stride_h = c.stride_h;
        g.stride_b = c.stride_b;
    }
    if (c.out_stride_b == 0 && c.out_stride_h == 0 && c.out_stride_n == 0) {
        g.ostride_b = g.stride_b;
        g.ostride_h = g.stride_h;
        g.ostride_n = g.stride_n;
    } else {
        if (c.out_stride_n < c.head_dim || c.out_stride_h <= 0 || c.out_stride_b <= 0) return DA2_ERR_INVALID_ARG;
        g.ostride_b = c.out_stride_b;
        g.ostride_h = c.out_stride_h;
        g.ostride_n = c.out_stride_n;
    }
    g.tau = c.softmax_scale > 0.0 ? c.softmax_scale : 1.0 / std::sqrt((double)c.head_dim);

    // workspace layout
    const uint64_t B = (uint64_t)bh, N = (uint64_t)nb, T = DA2_TILE, P = DA2_DPAD;
    da2::Layout L{};
    uint64_t off = 0;
    auto take = [&](uint64_t bytes) { uint64_t o = off; off = align256(off + bytes); return o; };
    L.pool = take(4 * B * N * P * 8);
    L.k8 = take(B * N * T * P);
    L.q8 = take(B * N * T * P);
    L.v8t = take(B * N * P * T);
    L.e8 = take(3 * B * N);
    L.q4 = take(B * N * T * P / 2);
    L.k4 = take(B * N * T * P / 2);
    L.v4t = take(B * N * P * T / 2);
    L.sq4 = take(B * N * T * (P / 32));
    L.sk4 = take(B * N * T * (P / 32));
    L.sv4t = take(B * N * P * (T / 32));
    L.scores = take(2 * B * N * N * 8);
    L.labels = take(B * N * N);
    L.hi = take(B * N * (uint64_t)(g.n_hi > 0 ? g.n_hi : 1) * 4);
    L.lo = take(B * N * (uint64_t)(g.n_lo > 0 ? g.n_lo : 1) * 4);
    L.status = take(16);
    L.bias = take((N + 1) * T * 4);   // row N: a tile with no keys (all -inf)
    L.total = off;

    da2_plan_t* p = new (std::nothrow) da2_plan_t;
    if (!p) return DA2_ERR_INVALID_ARG;
    p->cfg = c;
    p->geo = g;
    p->ws = L;
    *out = p;
    return DA2_OK;
}

extern "C" void da2_plan_destroy(da2_plan_t* plan) { delete plan; }

extern "C" da2_status da2_plan_info(const da2_plan_t* plan, da2_plan_info_t* out) {
    if (!plan || !out) return DA2_ERR_INVALID_ARG;
    const da2::Geo& g = plan->geo;
    const da2::Layout& L = plan->ws;
    da2_plan_info_t i{};
    i.n_blocks = g.n_blocks;
    i.block_size = g.block_size;
    i.n_wy = g.n_wy;
    i.n_wx = g.n_wx;
    i.n_hi = g.n_hi;
    i.n_lo = g.n_lo;
    i.tokens = g.tokens;
    i.slots = (int64_t)g.n_blocks * g.block_size;
    i.tau = g.tau;
    i.workspace_bytes = L.total;
    i.n_full = g.n_full;
    i.flags = plan->cfg.flags;
    i.off_pool = L.pool;
    i.off_k8 = L.k8;
    i.off_v8t = L.v8t;
    i.off_e8 = L.e8;
    i.off_q4 = L.q4;
    i.off_k4 = L.k4;
    i.off_v4t = L.v4t;
    i.off_sq4 = L.sq4;
    i.off_sk4 = L.sk4;
    i.off_sv4t = L.sv4t;
    i.off_scores = L.scores;
    i.off_labels = L.labels;
    i.off_hi = L.hi;
    i.off_lo = L.lo;
    i.off_status = L.status;
    i.off_q8 = L.q8;
    i.off_bias = L.bias;
    *out = i;
    return DA2_OK;
}

extern "C" const char* da2_status_string(da2_status s) {
    switch (s) {
        case DA2_OK: return "ok";
        case DA2_ERR_INVALID_ARG: return "invalid argument";
        case DA2_ERR_UNSUPPORTED: return "unsupported configuration";
        case DA2_ERR_WORKSPACE: return "workspace too small or misaligned";
        case DA2_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}
