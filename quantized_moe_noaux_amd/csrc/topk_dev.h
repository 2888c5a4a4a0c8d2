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
    int rank[kMaxExperts];       // rank of each candidate among the kept
    int sel_e[kMaxTopK];
    double sel_s[kMaxTopK];
};

// Block-wide noaux_tc routing of one token (every thread of the block calls
// it; blockDim.x >= 64).  The selection is a parallel rank count:
//   rank(e) = #{kept candidates e' with c' > c, or c' == c and e' < e}
// and e is selected at position rank(e) when that is below k.  Every phase
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
        L.rank[e] = 0;
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
    // rank counting: one item = (candidate, kept group scanned)
    const int nk = L.nkept, ncand = nk * m;
    for (int it = tid; it < ncand * nk; it += nt) {
        const int ci = it % ncand, gi = it / ncand;
        const int e = L.kept[ci / m] * m + (ci % m);
        const uint64_t ke = L.key[e];
        const int base = L.kept[gi] * m;
        int cnt = 0;
        for (int j0 = 0; j0 < m; j0 += 8) {
            uint64_t kj[8];
#pragma unroll
            for (int j = 0; j < 8; j++) kj[j] = (j0 + j < m) ? L.key[base + j0 + j] : 0ull;
#pragma unroll
            for (int j = 0; j < 8; j++)
                cnt += (kj[j] > ke) || (kj[j] == ke && base + j0 + j < e && j0 + j < m);
        }
        if (cnt) atomicAdd(&L.rank[e], cnt);
    }
    __syncthreads();
    for (int ci = tid; ci < ncand; ci += nt) {
        const int e = L.kept[ci / m] * m + (ci % m);
        const int r = L.rank[e];
        if (r < rc.k) { L.sel_e[r] = e; L.sel_s[r] = L.s[e]; }
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
