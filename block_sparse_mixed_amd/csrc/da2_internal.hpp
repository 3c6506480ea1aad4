// Internal declarations shared by the host plan code and the kernel launchers.
#pragma once

#include <cstdint>

#include "da2.h"

namespace da2 {

// Geometry and sizes every kernel needs, passed by value.
struct Geo {
    int32_t frames, grid_h, grid_w, win_h, win_w;
    int32_t n_wy, n_wx, n_blocks, block_size, head_dim, heads, bh;
    // packed edge windows: pack != 0; fwy x fwx full windows a frame, n_full
    // of them in all; edge_frame partial-window tokens a frame, edge_total in all
    int32_t pack, fwy, fwx, n_full, edge_frame, edge_total;
    int32_t n_hi, n_lo;
    int64_t tokens;
    int64_t stride_b, stride_h, stride_n;
    int64_t ostride_b, ostride_h, ostride_n;   // of out
    double tau;
};

struct Layout {
    uint64_t pool, k8, q8, v8t, e8, q4, k4, v4t, sq4, sk4, sv4t, scores, labels, hi, lo, status, bias;
    uint64_t total;
};

}  // namespace da2

struct da2_plan_s {
    da2_config cfg;
    da2::Geo geo;
    da2::Layout ws;
};
