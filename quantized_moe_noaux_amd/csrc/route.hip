// Router and activation quantiser kernels.
//
// Router: DeepSeek-V3-style sigmoid router with noaux_tc (GeekNews #31297,
// implemented features; wpnews.pro spec table: 8 of 256 experts per token).
// Logits x.W_e accumulate in fp64 (each fp32 x fp32 product is exact in
// fp64), and the sigmoid and every comparison are fp64 too, so that the
// selected experts do not depend on the summation order.
#include "moe_dev.h"
#include "moe_internal.h"
#include "topk_dev.h"

namespace moe {

bool route_cfg(const moe_shape_t &s, RouteCfg &rc)
{
    const int E = s.n_experts, G = s.n_group, m = E / G;
    int lo = (E + kWave - 1) / kWave;
    for (int epl = lo; epl <= 8; epl++) {
        if (m % epl) continue;
        int lpg = m / epl;
        if (lpg & (lpg - 1)) continue;
        rc.E = E; rc.G = G; rc.tg = s.topk_group; rc.k = s.top_k;
        rc.epl = epl; rc.lpg = lpg; rc.rsf = s.routed_scaling_factor;
        rc.top_p = top_p_on(s) ? s.routed_top_p : 0.f;
        return true;
    }
    return false;
}

// ---------------------------------------------------------------- logits, small T
// Block b < E computes z[t][b] for all T <= 8 tokens; blocks >= E quantise x.
// With ng != nullptr the input is RMSNorm(x) with weight ng: every block
// normalises the rows it reads itself (a block-wide fp64 sum of squares per
// token, the same arithmetic as the RMSNorm kernel, so the values equal that
// kernel's output) and the normalised row never goes through memory.  The
// host only passes ng for H <= 8192, H % 4 == 0 and 16-byte aligned x, ng.
// With la_logits != nullptr (router lookahead of a decode stack), blocks
// E .. 2E-1 compute the next layer's logits the same way on the same x, with
// that layer's router weights la_gate_w and norm weight la_ng.
__global__ __launch_bounds__(256) void k_router_logits_small(
    const float *__restrict__ x, int T, int H, const float *__restrict__ gate_w_l, int E,
    double *__restrict__ logits_l, int8_t *__restrict__ xq, float *__restrict__ xd,
    const float *__restrict__ ng_l, double eps, const float *__restrict__ la_gate_w,
    const float *__restrict__ la_ng, double *__restrict__ la_logits)
{
    __shared__ double red[4][kGemvMaxT];
    __shared__ double nred[kGemvMaxT][4];
    const int tid = threadIdx.x;
    const int n4 = H / 4;
    const int nlog = la_logits ? 2 * E : E;  // logit blocks
    if ((int)blockIdx.x < nlog) {
        const bool la = (int)blockIdx.x >= E;
        const int e = la ? (int)blockIdx.x - E : (int)blockIdx.x;
        const float *gate_w = la ? la_gate_w : gate_w_l;
        const float *ng = la ? la_ng : ng_l;
        double *logits = la ? la_logits : logits_l;
        double acc[kGemvMaxT];
#pragma unroll
        for (int t = 0; t < kGemvMaxT; t++) acc[t] = 0.0;
        const float4 *wr = reinterpret_cast<const float4 *>(gate_w + (size_t)e * H);
        constexpr int kPer = kNormPer;  // float4s per thread per pass: all loads issued before use
        if (ng) {
            float4 w[kPer], gv[kPer];
#pragma unroll
            for (int j = 0; j < kPer; j++) {
                w[j] = load4_masked(wr, tid + 256 * j, n4);
                gv[j] = load4_masked(reinterpret_cast<const float4 *>(ng), tid + 256 * j, n4);
            }
#pragma unroll
            for (int t = 0; t < kGemvMaxT; t++) {
                if (t < T) {
                    float4 v[kNormPer];
                    load_row_regs(x + (size_t)t * H, n4, v);
                    const double r = row_rstd(v, H, eps, nred[t]);
#pragma unroll
                    for (int j = 0; j < kPer; j++) {
                        // masked-off lanes hold zeros in w, v and gv
                        const float4 n = norm4(v[j], r, gv[j]);
                        acc[t] = fma((double)w[j].x, (double)n.x, acc[t]);
                        acc[t] = fma((double)w[j].y, (double)n.y, acc[t]);
                        acc[t] = fma((double)w[j].z, (double)n.z, acc[t]);
                        acc[t] = fma((double)w[j].w, (double)n.w, acc[t]);
                    }
                }
            }
        } else {
            for (int base = 0; base < n4; base += 256 * kPer) {
                float4 w[kPer];
#pragma unroll
                for (int j = 0; j < kPer; j++) w[j] = load4_masked(wr, base + tid + 256 * j, n4);
#pragma unroll
                for (int t = 0; t < kGemvMaxT; t++) {
                    if (t < T) {
                        const float4 *xr = reinterpret_cast<const float4 *>(x + (size_t)t * H);
                        float4 v[kPer];
#pragma unroll
                        for (int j = 0; j < kPer; j++) v[j] = load4_masked(xr, base + tid + 256 * j, n4);
#pragma unroll
                        for (int j = 0; j < kPer; j++) {
                            acc[t] = fma((double)w[j].x, (double)v[j].x, acc[t]);
                            acc[t] = fma((double)w[j].y, (double)v[j].y, acc[t]);
                            acc[t] = fma((double)w[j].z, (double)v[j].z, acc[t]);
                            acc[t] = fma((double)w[j].w, (double)v[j].w, acc[t]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < kGemvMaxT; t++) {
            if (t < T) {
                double v = wave_sum_d(acc[t]);
                if (lane_id() == 0) red[wave_id()][t] = v;
            }
        }
        __syncthreads();
        if (tid < T) logits[(size_t)tid * E + e] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
        return;
    }
    // quantiser part: 8 lanes per block of 32
    const float *ng = ng_l;
    const int nb = H / 32;
    const int g = ((int)blockIdx.x - nlog) * 256 + tid;
    const int b = g >> 3, sub = g & 7;
    const bool live = b < T * nb;
    float4 v = live ? reinterpret_cast<const float4 *>(x + (size_t)b * 32)[sub] : make_float4(0, 0, 0, 0);
    if (ng) {
        // the tokens this block's 32 blocks of 32 fall in (block-uniform bounds)
        const int b0 = ((int)blockIdx.x - nlog) * 32;
        const int b1 = min(b0 + 31, T * nb - 1);
        double r = 0.0;
        for (int t = b0 / nb; t <= b1 / nb; t++) {
            float4 row[kNormPer];
            load_row_regs(x + (size_t)t * H, n4, row);
            const double rt = row_rstd(row, H, eps, nred[t]);
            if (live && b / nb == t) r = rt;
        }
        if (live) v = norm4(v, r, reinterpret_cast<const float4 *>(ng)[(b % nb) * 8 + sub]);
    }
    float d;
    uint32_t packed = quant_block8(v, d);
    if (live) {
        reinterpret_cast<uint32_t *>(xq + (size_t)b * 32)[sub] = packed;
        if (sub == 0) xd[b] = d;
    }
}

int launch_router_logits(const float *x, int T, int H, const float *gate_w, int E, double *logits,
                         int8_t *xq, float *xd, const float *ng, double eps, hipStream_t st,
                         const float *la_gate_w, const float *la_ng, double *la_logits)
{
    if (ng && !router_norms_input(x, ng, H)) return (int)hipErrorInvalidValue;
    if (la_logits && (!la_gate_w || !la_ng || !ng || !router_norms_input(x, la_ng, H)))
        return (int)hipErrorInvalidValue;
    const int qblocks = xq ? (T * (H / 32) * 8 + 255) / 256 : 0;
    const int nlog = la_logits ? 2 * E : E;
    k_router_logits_small<<<nlog + qblocks, 256, 0, st>>>(x, T, H, gate_w, E, logits, xq, xd, ng, eps, la_gate_w,
                                                          la_ng, la_logits);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------- logits, any T
// fp64 matrix cores: v_mfma_f64_16x16x4f64 on x (tokens) and gate_w
// (experts), both widened from fp32 in registers (exact).  One wave owns 32
// tokens x 64 experts over one of `ksplit` equal K slices; the partial sums
// land in part[slice][T][E] and the top-k kernel adds the slices in order.
// Lane l feeds row / column l%16 of each 16x16 tile with k = 4*(l/16) + s of
// every 16-wide K block (s = 0..3: one float4 per lane and operand); the
// result of lane l, register v is row l/16 + 4v, column l%16.
typedef double v4d __attribute__((ext_vector_type(4)));

int router_ksplit(int T, int H, int E)
{
    if (T <= kGemvMaxT) return 1;
    const long tiles = (long)((T + 31) / 32) * ((E + 63) / 64);
    const int kb = H / 16;
    int ks = 1;
    while (ks < 32 && tiles * ks < 2048 && kb % (2 * ks) == 0 && kb / (2 * ks) >= 4) ks *= 2;
    return ks;
}

__device__ __forceinline__ float f4c(const float4 &v, int s)
{
    return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

__global__ __launch_bounds__(256) void k_router_logits_mfma(const float *__restrict__ x, int T, int H,
                                                            const float *__restrict__ gate_w, int E, int ksplit,
                                                            double *__restrict__ part)
{
    const int l = lane_id();
    const int wv = blockIdx.x * 4 + wave_id();
    const int et = (E + 63) / 64, tt = (T + 31) / 32;
    const int ks = wv % ksplit, te = wv / ksplit;
    const int ei = te % et, ti = te / et;
    if (ti >= tt) return;
    const int t0 = ti * 32, e0 = ei * 64;
    const int kq = H / ksplit, kbeg = ks * kq;
    const int r = l & 15, g = l >> 4;
    const float *pa[2], *pb[4];
    bool va[2], vb[4];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int t = t0 + 16 * i + r;
        va[i] = t < T;
        pa[i] = x + (size_t)(va[i] ? t : 0) * H + kbeg + 4 * g;
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int e = e0 + 16 * j + r;
        vb[j] = e < E;
        pb[j] = gate_w + (size_t)(vb[j] ? e : 0) * H + kbeg + 4 * g;
    }
    v4d acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = (v4d){0.0, 0.0, 0.0, 0.0};
    // three register sets: the K block being multiplied and the next two in
    // flight (one wave per SIMD pair: the loads' latency is not hidden by
    // other waves)
    // Loads are unconditional, so they issue as plain dwordx4 loads with
    // partial waits: a row past T or E reads row 0 (its results are never
    // stored, and rows do not mix in the product), and a block past the
    // slice end re-reads the last block (it is never multiplied).
    float4 a[3][2], b[3][4];
    auto fetch = [&](int set, int kk) {
        const int kc = kk < kq ? kk : kq - 16;
#pragma unroll
        for (int i = 0; i < 2; i++) a[set][i] = *reinterpret_cast<const float4 *>(pa[i] + kc);
#pragma unroll
        for (int j = 0; j < 4; j++) b[set][j] = *reinterpret_cast<const float4 *>(pb[j] + kc);
    };
    auto mul = [&](int set) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            double da[2], db[4];
#pragma unroll
            for (int i = 0; i < 2; i++) da[i] = (double)f4c(a[set][i], s);
#pragma unroll
            for (int j = 0; j < 4; j++) db[j] = (double)f4c(b[set][j], s);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(da[i], db[j], acc[i][j], 0, 0, 0);
        }
    };
    fetch(0, 0);
    fetch(1, 16);
    int kk = 0;
    // kq is a multiple of 16; unrolled by three so the register sets stay static
    for (; kk + 48 <= kq; kk += 48) {
        fetch(2, kk + 32);
        mul(0);
        fetch(0, kk + 48);
        mul(1);
        fetch(1, kk + 64);
        mul(2);
    }
    if (kk < kq) mul(0);
    if (kk + 16 < kq) mul(1);
    double *o = part + (size_t)ks * T * E;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int t = t0 + 16 * i + g + 4 * v, e = e0 + 16 * j + r;
                if (t < T && e < E) o[(size_t)t * E + e] = acc[i][j][v];
            }
}

int launch_router_logits_mfma(const float *x, int T, int H, const float *gate_w, int E, int ksplit, double *part,
                              hipStream_t st)
{
    const long waves = (long)((T + 31) / 32) * ((E + 63) / 64) * ksplit;
    k_router_logits_mfma<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(x, T, H, gate_w, E, ksplit, part);
    return (int)hipGetLastError();
}

// one wave per token; the logits are the sum of `nparts` slices.  A wave
// past the last token routes the last token again and stores nothing.
__global__ __launch_bounds__(256) void k_topk(const RouteCfg rc, const double *__restrict__ logits, int nparts,
                                              const float *__restrict__ bias, int T,
                                              int32_t *__restrict__ idx, float *__restrict__ w)
{
    const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(wave_id()), tr = min(t, T - 1);
    const WaveSel ws = wave_topk(rc, logits + (size_t)tr * rc.E, (size_t)T * rc.E, nparts, bias, rc.k);
    const int lane = lane_id();
    if (t < T && lane < rc.k) {
        idx[(size_t)t * rc.k + lane] = ws.e;
        w[(size_t)t * rc.k + lane] = ws.w;
    }
}

int launch_topk(const RouteCfg &rc, const double *logits, int nparts, const float *bias, int T, int32_t *idx,
                float *w, hipStream_t st)
{
    k_topk<<<(T + 3) / 4, 256, 0, st>>>(rc, logits, nparts, bias, T, idx, w);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------- quantiser
__global__ __launch_bounds__(256) void k_quant(const float *__restrict__ x, long nblocks,
                                               int8_t *__restrict__ q, float *__restrict__ d)
{
    const long g = (long)blockIdx.x * 256 + threadIdx.x;
    const long b = g >> 3;
    const int sub = (int)(g & 7);
    const bool live = b < nblocks;
    float4 v = live ? reinterpret_cast<const float4 *>(x + (size_t)b * 32)[sub] : make_float4(0, 0, 0, 0);
    float db;
    uint32_t packed = quant_block8(v, db);
    if (live) {
        reinterpret_cast<uint32_t *>(q + (size_t)b * 32)[sub] = packed;
        if (sub == 0) d[b] = db;
    }
}

int launch_quant(const float *x, int T, int D, int8_t *q, float *d, hipStream_t st)
{
    const long nb = (long)T * (D / 32);
    const long blocks = (nb * 8 + 255) / 256;
    if (!blocks) return 0;
    k_quant<<<(unsigned)blocks, 256, 0, st>>>(x, nb, q, d);
    return (int)hipGetLastError();
}

} // namespace moe
