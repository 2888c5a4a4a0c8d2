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

// Lane exchanges for the group phase.  DPP moves (quad_perm, row mirrors)
// stay inside the VALU; a cross-lane permute through the LDS crossbar costs
// a round trip of ~100 cycles per step on MI355X.
template <int CTRL> __device__ __forceinline__ double dpp_d(double v)
{
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double readlane_d(double v, int l)
{
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
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

// LDS scratch of block_topk.  Keys are stored per group at a stride of
// mpad = m rounded up to 8 (zero keys in the padding), so the in-group rank
// loop reads whole 8-key steps with no bounds checks: a zero key never
// outranks a real one.
struct __align__(16) TopkLds {
    // the last entry of s, c and key is a dump slot: a lane without an
    // expert stores there, so its loads and stores need no branch
    double s[kMaxExperts + 1];                       // sigmoid scores
    double c[kMaxExperts + 1];                       // c = s + bias
    uint64_t key[kMaxExperts + 7 * kMaxGroups + 1];  // order keys, group-strided
    uint64_t fkey[kMaxExperts];                  // finalists' keys
    int fe[kMaxExperts];                         // finalists' experts
    int frank[kMaxExperts];                      // finalists' ranks among the finalists
    int kept[kMaxGroups];                        // kept groups, ascending
    int nkept;
    int sel_e[kMaxTopK];
    double sel_s[kMaxTopK];
};

// Number of keys among the 8 at p that outrank key ke at position pos
// (position j outranks if its key is larger, or equal with j < pos).
__device__ __forceinline__ int outrank8(const uint64_t *p, int j0, uint64_t ke, int pos)
{
    const ulonglong2 *q = reinterpret_cast<const ulonglong2 *>(p);
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const ulonglong2 v = q[u];
        cnt += (v.x > ke) || (v.x == ke && j0 + 2 * u < pos);
        cnt += (v.y > ke) || (v.y == ke && j0 + 2 * u + 1 < pos);
    }
    return cnt;
}

// Block-wide noaux_tc routing of one token (every thread of the block calls
// it; nt >= 64 threads take part).  Every phase spreads its work over many lanes with
// independent loads: on MI355X a dependent LDS or cross-lane round trip costs
// ~100 cycles, so serial chains, not arithmetic, set the latency of this step.
//   1. s, c = s + bias and the order key of c for every expert (all logit
//      loads issued before any arithmetic);
//   2. one wave: group score = sum of the two largest c (lane l holds the
//      experts epl*l ..; a group spans lpg lanes, merged by DPP), and the
//      topk_group best groups (score desc, index asc) are kept;
//   3. in-group rank of every candidate of a kept group; only a candidate
//      with in-group rank < k can be among the top k, so each kept group
//      has exactly min(m, k) finalists, stored at (kept slot, in-group rank);
//   4. rank of every finalist among the finalists: for a finalist in the top
//      k it equals its rank among all candidates (every candidate above it is
//      a finalist too), and one outside the top k has rank >= k there too.
//      Equal keys rank by position, which is expert order (kept groups
//      ascend, and in-group ranks order equal keys by expert index), so a
//      tie goes to the lower expert index.  The rank is the in-group rank
//      plus, per other kept group, the length of that group's run of
//      finalists that outrank it: a group's finalists sit in outrank order,
//      so a binary search finds the run;
//   5. the selected s normalised to sum one, times routed_scaling_factor;
//      with adaptive top-p (rc.top_p in (0, 1)) only the shortest prefix of
//      the selection whose share of the summed s reaches p is kept and
//      renormalised, and the dropped slots read expert -1, weight 0.
// All scores and comparisons are fp64 (order keys compare as the doubles).
//   zt: the token's logits, as the sum of nparts slices pstride apart
//   (added in slice order)
//   tid, nt: this thread's index among the nt threads (a multiple of 64)
//   that route this token; several groups of a workgroup may route
//   different tokens at once, each with its own L, since the barriers are
//   workgroup-wide and every group passes the same ones.
__device__ __forceinline__ void block_topk(const RouteCfg rc, const double *__restrict__ zt, size_t pstride, int nparts,
                           const float *__restrict__ bias, int *sel_e, float *sel_w, TopkLds &L, int tid,
                           int nt)
{
    const int lane = lane_id();
    const int E = rc.E, G = rc.G, m = E / G, k = rc.k;
    const int mpad = (m + 7) & ~7;
    const int kdump = kMaxExperts + 7 * kMaxGroups;
    for (int e0 = 0; e0 < E; e0 += 2 * nt) {
        // both experts' loads at clamped indices, unconditionally (one round
        // trip); a lane past E computes on a duplicate and stores it in the
        // dump slots
        const int ea = e0 + tid, eb = e0 + nt + tid;
        const int ca = min(ea, E - 1), cb = min(eb, E - 1);
        double za = zt[ca], zb = zt[cb];
        const float ba = bias[ca], bb = bias[cb];
        for (int p = 1; p < nparts; p++) {
            za += zt[p * pstride + ca];
            zb += zt[p * pstride + cb];
        }
        const double sa = 1.0 / (1.0 + exp(-za)), cva = sa + (double)ba;
        const double sb = 1.0 / (1.0 + exp(-zb)), cvb = sb + (double)bb;
        const int da = ea < E ? ea : kMaxExperts, db = eb < E ? eb : kMaxExperts;
        L.s[da] = sa;
        L.c[da] = cva;
        L.key[ea < E ? (ea / m) * mpad + ea % m : kdump] = order_key(cva);
        L.s[db] = sb;
        L.c[db] = cvb;
        L.key[eb < E ? (eb / m) * mpad + eb % m : kdump] = order_key(cvb);
    }
    for (int i = tid; i < G * (mpad - m); i += nt) L.key[(i / (mpad - m)) * mpad + m + i % (mpad - m)] = 0ull;
    __syncthreads();
    if (tid < 64) {
        const int epl = rc.epl, lpg = rc.lpg;
        // all eight reads issued at once (clamped in bounds, masked after),
        // then a branch-free top-2 insertion
        double cvs[8];
#pragma unroll
        for (int j = 0; j < 8; j++) cvs[j] = L.c[min(lane * epl + j, E - 1)];
        double b1 = -INFINITY, b2 = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const double cv = (j < epl && lane * epl + j < E) ? cvs[j] : -INFINITY;
            b2 = fmax(b2, fmin(b1, cv));
            b1 = fmax(b1, cv);
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
        const bool keep = g < G && lane % lpg == 0 && grank < rc.tg;
        const unsigned long long kb = __ballot(keep);
        if (keep) L.kept[__popcll(kb & ((1ull << lane) - 1))] = g;
        if (lane == 0) L.nkept = __popcll(kb);
    }
    __syncthreads();
    const int nk = L.nkept, f1 = m < k ? m : k, nf = nk * f1;
    for (int ci = tid; ci < nk * m; ci += nt) {
        const int slot = ci / m, r = ci - slot * m, g = L.kept[slot];
        const uint64_t *gk = L.key + g * mpad;
        const uint64_t ke = gk[r];
        int cnt = 0;
        for (int j = 0; j < mpad; j += 8) cnt += outrank8(gk + j, j, ke, r);
        if (cnt < f1) {
            L.fkey[slot * f1 + cnt] = ke;
            L.fe[slot * f1 + cnt] = g * m + r;
            L.frank[slot * f1 + cnt] = 0;
        }
    }
    __syncthreads();
    int top = 1;  // largest power of two <= f1
    while (2 * top <= f1) top *= 2;
    for (int it = tid; it < nf * nk; it += nt) {
        const int fi = it / nk, b = it - fi * nk, ga = fi / f1;
        int cnt;
        if (b == ga) {
            cnt = fi - ga * f1;
        } else {
            // group b's entries at positions before fi's group outrank it on
            // equal keys too
            const uint64_t kx = L.fkey[fi], *gb = L.fkey + b * f1;
            cnt = 0;
            for (int st = top; st > 0; st >>= 1) {
                const int j = cnt + st - 1;
                if (j < f1) {
                    const uint64_t ky = gb[j];
                    if (ky > kx || (ky == kx && b < ga)) cnt += st;
                }
            }
        }
        atomicAdd(&L.frank[fi], cnt);
    }
    __syncthreads();
    for (int fi = tid; fi < nf; fi += nt) {
        const int r = L.frank[fi];
        if (r < k) {
            const int e = L.fe[fi];
            L.sel_e[r] = e;
            L.sel_s[r] = L.s[e];
        }
    }
    __syncthreads();
    if (tid < k) {
        double sum = 0.0;
        for (int i = 0; i < k; i++) sum += L.sel_s[i];
        int kept = k;
        if (rc.top_p > 0.f) {
            // adaptive top-p: the shortest prefix whose share of the summed s
            // reaches p (shares added in slot order), renormalised
            const double p = (double)rc.top_p;
            double cum = 0.0;
            kept = 0;
            while (kept < k) {
                cum += L.sel_s[kept] / sum;
                kept++;
                if (cum >= p) break;
            }
            sum = 0.0;
            for (int i = 0; i < kept; i++) sum += L.sel_s[i];
        }
        sel_e[tid] = (tid < kept) ? L.sel_e[tid] : -1;
        sel_w[tid] = (tid < kept) ? (float)(L.sel_s[tid] / sum * (double)rc.rsf) : 0.f;
    }
    __syncthreads();
}

// the whole workgroup routes one token
__device__ __forceinline__ void block_topk(const RouteCfg rc, const double *__restrict__ zt, size_t pstride,
                                           int nparts, const float *__restrict__ bias, int *sel_e, float *sel_w,
                                           TopkLds &L)
{
    block_topk(rc, zt, pstride, nparts, bias, sel_e, sel_w, L, threadIdx.x, blockDim.x);
}

} // namespace moe
