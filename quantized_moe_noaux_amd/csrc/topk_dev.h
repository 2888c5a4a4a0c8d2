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

// LDS scratch of block_topk
struct TopkLds {
    uint64_t key[kMaxExperts];   // order key of c = s + bias
    double c[kMaxExperts];
    double s[kMaxExperts];       // sigmoid scores
    double gs[kMaxGroups];       // group scores
    int kept[kMaxGroups];        // kept groups, ascending
    int nkept;
    uint64_t ckey[kMaxExperts];  // keys of the kept candidates, in expert order
    int crank[2][kMaxExperts];   // partial ranks of the kept candidates
    int sel_e[kMaxTopK];
    double sel_s[kMaxTopK];
};

// Block-wide noaux_tc routing of one token (every thread of the block calls
// it; blockDim.x >= 64).  The selection is a parallel rank count:
//   rank(e) = #{kept candidates e' with c' > c, or c' == c and e' < e}
// and e is selected at position rank(e) when that is below k (key 0 = a
// padding entry never outranks a real one: real keys are above 0).  Every phase
// spreads its work over many lanes with independent loads: on MI355X a
// dependent LDS or cross-lane round trip costs ~100 cycles, so serial
// chains, not arithmetic, set the latency of this step.  All scores and
// comparisons are fp64.
//   zt: the token's logits, as the sum of nparts slices pstride apart
//   (added in slice order)
__device__ void block_topk(const RouteCfg rc, const double *__restrict__ zt, size_t pstride, int nparts,
                           const float *__restrict__ bias, int *sel_e, float *sel_w, TopkLds &L)
{
    const int tid = threadIdx.x, nt = blockDim.x, lane = lane_id();
    const int E = rc.E, G = rc.G, m = E / G;
    for (int e = tid; e < E; e += nt) {
        double z = zt[e];
        for (int p = 1; p < nparts; p++) z += zt[p * pstride + e];
        const double sv = 1.0 / (1.0 + exp(-z));
        const double cv = sv + (double)bias[e];
        L.s[e] = sv;
        L.c[e] = cv;
        L.key[e] = order_key(cv);
    }
    __syncthreads();
    if (tid < 64) {
        // group score = sum of the two largest c: lpg lanes per group (a power
        // of two), each scanning <= 8 experts, then a lane butterfly
        int lpg = 1;
        while (lpg * 2 * G <= 64) lpg <<= 1;
        const int g = lane / lpg, sub = lane % lpg;
        double b1 = -INFINITY, b2 = -INFINITY;
        if (g < G) {
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const int r = sub + lpg * j;
                if (r < m) {
                    const double cv = L.c[g * m + r];
                    if (cv > b1) { b2 = b1; b1 = cv; }
                    else if (cv > b2) b2 = cv;
                }
            }
        }
        for (int o = 1; o < lpg; o <<= 1) {
            const double o1 = __shfl_xor(b1, o), o2 = __shfl_xor(b2, o);
            const double n2 = fmax(fmin(b1, o1), fmax(b2, o2));
            b1 = fmax(b1, o1);
            b2 = n2;
        }
        const double gsv = (m >= 2) ? b1 + b2 : b1;
        // rank of each group among the G (score desc, index asc)
        int grank = 0;
        for (int h = 0; h < G; h++) {
            const double o = __shfl(gsv, h * lpg);
            grank += (o > gsv) || (o == gsv && h < g);
        }
        const bool keep = g < G && sub == 0 && grank < rc.tg;
        const unsigned long long kb = __ballot(keep);
        if (keep) L.kept[__popcll(kb & ((1ull << lane) - 1))] = g;
        if (lane == 0) L.nkept = __popcll(kb);
    }
    __syncthreads();
    // Candidates = the experts of the kept groups; kept groups ascend, so
    // candidate order is expert order and a tie goes to the lower position.
    // rank(ci) = #{j : key_j > key_ci, or key_j == key_ci and j < ci}, counted
    // by two threads per candidate over halves of j (broadcast LDS reads, no
    // atomics) and summed in a fixed order.
    const int nk = L.nkept, ncand = nk * m;
    for (int ci = tid; ci < ncand; ci += nt) L.ckey[ci] = L.key[L.kept[ci / m] * m + ci % m];
    __syncthreads();
    const int split = (2 * ncand <= nt) ? 2 : 1, half = ncand / split;
    for (int item = tid; item < ncand * split; item += nt) {
        const int ci = item % ncand, part = item / ncand;
        const int j0 = part * half, j1 = (part + 1 == split) ? ncand : j0 + half;
        const uint64_t ke = L.ckey[ci];
        int cnt = 0;
        for (int j = j0; j < j1; j += 8) {
            uint64_t kj[8];
#pragma unroll
            for (int u = 0; u < 8; u++) kj[u] = (j + u < j1) ? L.ckey[j + u] : 0ull;
#pragma unroll
            for (int u = 0; u < 8; u++) cnt += (kj[u] > ke) || (kj[u] == ke && j + u < ci);
        }
        L.crank[part][ci] = cnt;
    }
    __syncthreads();
    for (int ci = tid; ci < ncand; ci += nt) {
        const int r = L.crank[0][ci] + (split == 2 ? L.crank[1][ci] : 0);
        if (r < rc.k) {
            const int e = L.kept[ci / m] * m + ci % m;
            L.sel_e[r] = e;
            L.sel_s[r] = L.s[e];
        }
    }
    __syncthreads();
    if (tid < rc.k) {
        double sum = 0.0;
        for (int i = 0; i < rc.k; i++) sum += L.sel_s[i];
        sel_e[tid] = L.sel_e[tid];
        sel_w[tid] = (float)(L.sel_s[tid] / sum * (double)rc.rsf);
    }
    __syncthreads();
}

} // namespace moe
