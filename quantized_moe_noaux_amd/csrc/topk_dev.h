// noaux_tc expert selection for one token (device code).
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

// Order-preserving 64-bit key of a finite double (a larger double gets a
// larger key); key 0 is below every finite value and marks "excluded".
__device__ __forceinline__ uint64_t order_key(double v)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v + 0.0);  // -0 -> +0
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// (b1, b2) = the two largest of the multiset {b1, b2, o1, o2}, where b1 >= b2
// and o1 >= o2
__device__ __forceinline__ void merge_top2(double &b1, double &b2, double o1, double o2)
{
    const double n2 = fmax(fmin(b1, o1), fmax(b2, o2));
    b1 = fmax(b1, o1);
    b2 = n2;
}
template <int CTRL> __device__ __forceinline__ void dpp_top2(double &b1, double &b2)
{
    merge_top2(b1, b2, dpp_d<CTRL>(b1), dpp_d<CTRL>(b2));
}

// Largest value over the 64 lanes: one max per step with the DPP move fused
// into it inside each row of 16 lanes, then the four row maxima read into
// scalar registers (no LDS crossbar round trip).
template <int CTRL> __device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v)
{
    const uint32_t o = __builtin_amdgcn_update_dpp(0u, v, CTRL, 0xF, 0xF, false);
    return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = dpp_max_u32<0xB1>(v);   // lane ^ 1
    v = dpp_max_u32<0x4E>(v);   // lane ^ 2
    v = dpp_max_u32<0x141>(v);  // the other quad of 8
    v = dpp_max_u32<0x140>(v);  // the other half of 16
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}
// Mask of the lanes holding the largest 64-bit key: the upper halves first,
// the lower halves only when several lanes tie on the upper half.
__device__ __forceinline__ uint64_t wave_argmax_u64(uint64_t v)
{
    const uint32_t hi = (uint32_t)(v >> 32), mh = wave_max_u32(hi);
    uint64_t cand = __ballot(hi == mh);
    if (__popcll(cand) > 1) {  // uniform
        const uint32_t lo = (hi == mh) ? (uint32_t)v : 0u, ml = wave_max_u32(lo);
        cand = __ballot(hi == mh && (uint32_t)v == ml);
    }
    return cand;
}

// One routed selection as the calling wave's lanes hold it: lane i < k has
// the expert of rank i and its weight (-1 and 0 for a slot top-p dropped);
// last is the expert the final round picked (the same in every lane).
struct WaveSel {
    int e;
    float w;
    int last;
};

// noaux_tc routing of one token by one wave: all 64 lanes call it together
// (wave-uniform control flow), and it uses no LDS and no barrier, so the
// waves of a workgroup can route different tokens at once.  Lane l holds
// experts l*epl .. l*epl + epl - 1 in registers (EPL = epl, or 8 for any
// epl <= 8 with the unused entries masked).
//   1. s = sigmoid(z) and c = s + bias per expert, z being the sum of the
//      nparts logit slices pstride apart in slice order (all loads issued
//      at clamped indices first);
//   2. group score = sum of the two largest c of the group (a group spans
//      lpg lanes, merged by DPP moves and lane swaps); the topk_group best
//      groups (score desc, index asc) are kept;
//   3. k rounds of a wave-wide arg-max over the order keys of the kept
//      candidates: the largest key, and on equal keys the lowest lane and
//      then the lowest entry, which is the lowest expert index; the winner
//      drops out of later rounds.  Round r leaves its expert and s in lane r;
//   4. weights = selected s normalised to sum one (added in rank order),
//      times routed_scaling_factor; with adaptive top-p (rc.top_p in (0, 1))
//      the shortest rank prefix whose share of the sum reaches p is kept and
//      renormalised.
// With rounds < k only the first `rounds` ranks are found (no weights): the
// expert of rank rounds - 1 is `last`.
// Every score and comparison is fp64.
template <int EPL>
__device__ __forceinline__ WaveSel wave_topk_epl(const RouteCfg &rc, const double *__restrict__ zt, size_t pstride,
                                                 int nparts, const float *__restrict__ bias, int rounds)
{
    const int lane = lane_id();
    const int E = rc.E, G = rc.G, m = E / G, k = rc.k, lpg = rc.lpg;
    const int epl = (EPL == 8) ? rc.epl : EPL;
    double z[EPL];
    float bv[EPL];
#pragma unroll
    for (int j = 0; j < EPL; j++) {
        const int c = min(lane * epl + j, E - 1);
        z[j] = zt[c];
        bv[j] = bias[c];
    }
    for (int p = 1; p < nparts; p++) {
#pragma unroll
        for (int j = 0; j < EPL; j++) z[j] += zt[p * pstride + min(lane * epl + j, E - 1)];
    }
    double s[EPL], cv[EPL];
    bool valid[EPL];
#pragma unroll
    for (int j = 0; j < EPL; j++) {
        valid[j] = j < epl && lane * epl + j < E;
        if (j < epl) {  // uniform: only the generic form skips entries
            s[j] = 1.0 / (1.0 + exp(-z[j]));
            cv[j] = s[j] + (double)bv[j];
        } else {
            s[j] = 0.0;
            cv[j] = -INFINITY;
        }
    }
    double b1 = -INFINITY, b2 = -INFINITY;
#pragma unroll
    for (int j = 0; j < EPL; j++) {
        const double c = valid[j] ? cv[j] : -INFINITY;
        b2 = fmax(b2, fmin(b1, c));
        b1 = fmax(b1, c);
    }
    if (lpg > 1) dpp_top2<0xB1>(b1, b2);   // quad_perm [1,0,3,2]: lane ^ 1
    if (lpg > 2) dpp_top2<0x4E>(b1, b2);   // quad_perm [2,3,0,1]: lane ^ 2
    if (lpg > 4) dpp_top2<0x141>(b1, b2);  // row_half_mirror: the other quad of 8
    if (lpg > 8) dpp_top2<0x140>(b1, b2);  // row_mirror: the other half of 16
    for (int o = 16; o < lpg; o <<= 1) merge_top2(b1, b2, __shfl_xor(b1, o), __shfl_xor(b2, o));
    const double gsv = (m >= 2) ? b1 + b2 : b1;
    const int g = lane / lpg;
    int grank = 0;
    for (int h = 0; h < G; h++) {
        const double o = readlane_d(gsv, h * lpg);
        grank += (o > gsv) || (o == gsv && h < g);
    }
    const bool keep = g < G && grank < rc.tg;
    uint64_t key[EPL];
#pragma unroll
    for (int j = 0; j < EPL; j++) key[j] = (valid[j] && keep) ? order_key(cv[j]) : 0ull;

    int my_e = -1, last = -1;
    double my_s = 0.0, sum = 0.0;
    for (int r = 0; r < rounds; r++) {
        uint64_t bk = key[0];
        int bj = 0;
        double bs = s[0];
#pragma unroll
        for (int j = 1; j < EPL; j++)
            if (key[j] > bk) { bk = key[j]; bj = j; bs = s[j]; }
        // k <= kept candidates (checked on the host), so the maximum is a
        // real candidate's key; on equal keys the lowest lane wins
        const int w = __builtin_ctzll(wave_argmax_u64(bk));
        const int wj = __builtin_amdgcn_readlane(bj, w);
        const double se = readlane_d(bs, w);
        sum += se;
        last = w * epl + wj;
        if (lane == r) { my_e = last; my_s = se; }
#pragma unroll
        for (int j = 0; j < EPL; j++)
            if (lane == w && j == wj) key[j] = 0ull;
    }
    WaveSel o;
    o.last = last;
    if (rounds < k) {
        o.e = -1;
        o.w = 0.f;
        return o;
    }
    int kept = k;
    if (rc.top_p > 0.f) {
        const double p = (double)rc.top_p;
        double cum = 0.0;
        kept = 0;
        while (kept < k) {
            cum += readlane_d(my_s, kept) / sum;
            kept++;
            if (cum >= p) break;
        }
        sum = 0.0;
        for (int i = 0; i < kept; i++) sum += readlane_d(my_s, i);
    }
    o.e = (lane < kept) ? my_e : -1;
    o.w = (lane < kept) ? (float)(my_s / sum * (double)rc.rsf) : 0.f;
    return o;
}

// rounds = k: the whole selection; fewer: the expert of rank rounds - 1
__device__ __forceinline__ WaveSel wave_topk(const RouteCfg &rc, const double *__restrict__ zt, size_t pstride,
                                             int nparts, const float *__restrict__ bias, int rounds)
{
    if (rc.epl == 4) return wave_topk_epl<4>(rc, zt, pstride, nparts, bias, rounds);
    return wave_topk_epl<8>(rc, zt, pstride, nparts, bias, rounds);
}

} // namespace moe
