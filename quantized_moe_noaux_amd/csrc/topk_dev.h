// Wave-level noaux_tc expert selection for one token (device code).
//
// DeepSeek-V3-style sigmoid router with noaux_tc (GeekNews #31297,
// implemented features): s = sigmoid(z); the correction bias enters the
// selection only, c = s + bias; a group's score is the sum of its two
// largest c; the topk_group best groups are kept and the rest excluded; the
// top_k largest c among the kept experts are selected (ties to the lower
// index) and weighted by s normalised to sum one, times
// routed_scaling_factor.  All of it in fp64.
#pragma once
#include "moe_dev.h"
#include "moe_internal.h"

namespace moe {

// One wave routes one token.  Lane l holds experts l*epl .. l*epl+epl-1.
__device__ __forceinline__ void wave_topk(const RouteCfg rc, const double *__restrict__ zt, const float *__restrict__ bias,
                          int *sel_e, float *sel_w)
{
    const int lane = lane_id();
    const int m = rc.E / rc.G;
    double c[8], s[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        int e = lane * rc.epl + j;
        bool ok = j < rc.epl && e < rc.E;
        double z = ok ? zt[e] : 0.0;
        s[j] = 1.0 / (1.0 + exp(-z));
        c[j] = ok ? s[j] + (double)bias[e] : -INFINITY;
    }
    // group score: sum of the two largest biased scores of the group
    double b1 = -INFINITY, b2 = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        if (c[j] > b1) { b2 = b1; b1 = c[j]; }
        else if (c[j] > b2) b2 = c[j];
    }
    for (int o = 1; o < rc.lpg; o <<= 1) {
        double o1 = __shfl_xor(b1, o), o2 = __shfl_xor(b2, o);
        double n2 = fmax(fmin(b1, o1), fmax(b2, o2));
        b1 = fmax(b1, o1);
        b2 = n2;
    }
    const double gs = (m >= 2) ? b1 + b2 : b1;
    const int g = lane / rc.lpg;
    // keep the topk_group best groups (score desc, index asc)
    int rank = 0;
    for (int h = 0; h < rc.G; h++) {
        double o = __shfl(gs, h * rc.lpg);
        rank += (o > gs) || (o == gs && h < g);
    }
    const bool keep = g < rc.G && rank < rc.tg;
    double bv = -INFINITY;
    int bj = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        if (!keep) c[j] = -INFINITY;
        if (c[j] > bv) { bv = c[j]; bj = j; }
    }
    // k rounds of a wave arg-max (ties: lowest lane, then lowest j = lowest index)
    double sum = 0.0, my_s = 0.0;
    int my_e = 0;
    for (int i = 0; i < rc.k; i++) {
        double mx = wave_max_d(bv);
        unsigned long long hit = __ballot(bv == mx);
        int win = __ffsll((long long)hit) - 1;
        int wj = __shfl(bj, win);
        double sv = 0.0;
#pragma unroll
        for (int j = 0; j < 8; j++)
            if (j == bj) sv = s[j];
        sv = __shfl(sv, win);
        sum += sv;
        if (lane == i) { my_e = win * rc.epl + wj; my_s = sv; }
        if (lane == win) {
#pragma unroll
            for (int j = 0; j < 8; j++)
                if (j == bj) c[j] = -INFINITY;
            bv = -INFINITY;
            bj = 0;
#pragma unroll
            for (int j = 0; j < 8; j++)
                if (c[j] > bv) { bv = c[j]; bj = j; }
        }
    }
    if (lane < rc.k) {
        sel_e[lane] = my_e;
        sel_w[lane] = (float)(my_s / sum * (double)rc.rsf);
    }
}

} // namespace moe
