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
        return true;
    }
    return false;
}

// ---------------------------------------------------------------- logits, small T
// Block b < E computes z[t][b] for all T <= 8 tokens; blocks >= E quantise x.
__global__ __launch_bounds__(256) void k_router_logits_small(
    const float *__restrict__ x, int T, int H, const float *__restrict__ gate_w, int E,
    double *__restrict__ logits, int8_t *__restrict__ xq, float *__restrict__ xd)
{
    __shared__ double red[4][kGemvMaxT];
    const int tid = threadIdx.x;
    if ((int)blockIdx.x < E) {
        const int e = blockIdx.x;
        double acc[kGemvMaxT];
#pragma unroll
        for (int t = 0; t < kGemvMaxT; t++) acc[t] = 0.0;
        const float4 *wr = reinterpret_cast<const float4 *>(gate_w + (size_t)e * H);
        const int n4 = H / 4;
        constexpr int kPer = 8;  // float4s per thread per pass: all loads issued before use
        for (int base = 0; base < n4; base += 256 * kPer) {
            float4 w[kPer];
#pragma unroll
            for (int j = 0; j < kPer; j++) {
                const int i = base + tid + 256 * j;
                w[j] = (i < n4) ? wr[i] : make_float4(0, 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < kGemvMaxT; t++) {
                if (t < T) {
                    const float4 *xr = reinterpret_cast<const float4 *>(x + (size_t)t * H);
#pragma unroll
                    for (int j = 0; j < kPer; j++) {
                        const int i = base + tid + 256 * j;
                        if (i < n4) {
                            const float4 v = xr[i];
                            acc[t] = fma((double)w[j].x, (double)v.x, acc[t]);
                            acc[t] = fma((double)w[j].y, (double)v.y, acc[t]);
                            acc[t] = fma((double)w[j].z, (double)v.z, acc[t]);
                            acc[t] = fma((double)w[j].w, (double)v.w, acc[t]);
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
    const int nb = H / 32;
    const int g = ((int)blockIdx.x - E) * 256 + tid;
    const int b = g >> 3, sub = g & 7;
    const bool live = b < T * nb;
    float4 v = live ? reinterpret_cast<const float4 *>(x + (size_t)b * 32)[sub] : make_float4(0, 0, 0, 0);
    float d;
    uint32_t packed = quant_block8(v, d);
    if (live) {
        reinterpret_cast<uint32_t *>(xq + (size_t)b * 32)[sub] = packed;
        if (sub == 0) xd[b] = d;
    }
}

int launch_router_logits(const float *x, int T, int H, const float *gate_w, int E, double *logits,
                         int8_t *xq, float *xd, hipStream_t st)
{
    const int qblocks = xq ? (T * (H / 32) * 8 + 255) / 256 : 0;
    k_router_logits_small<<<E + qblocks, 256, 0, st>>>(x, T, H, gate_w, E, logits, xq, xd);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------- logits, any T
// 64 tokens x 64 experts per workgroup, 4 x 4 per thread, K in steps of 16
// staged in LDS already widened to fp64.
__global__ __launch_bounds__(256) void k_router_logits_tiled(
    const float *__restrict__ x, int T, int H, const float *__restrict__ gate_w, int E,
    double *__restrict__ logits)
{
    __shared__ double sx[16][64 + 2], sw[16][64 + 2];
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
    const int lr = tid >> 2, lk = (tid & 3) * 4;  // loader: row lr, k offset lk
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = 0.0;
    for (int k0 = 0; k0 < H; k0 += 16) {
        float4 xv = (t0 + lr < T) ? *reinterpret_cast<const float4 *>(x + (size_t)(t0 + lr) * H + k0 + lk)
                                  : make_float4(0, 0, 0, 0);
        float4 wv = (e0 + lr < E) ? *reinterpret_cast<const float4 *>(gate_w + (size_t)(e0 + lr) * H + k0 + lk)
                                  : make_float4(0, 0, 0, 0);
        sx[lk][lr] = xv.x; sx[lk + 1][lr] = xv.y; sx[lk + 2][lr] = xv.z; sx[lk + 3][lr] = xv.w;
        sw[lk][lr] = wv.x; sw[lk + 1][lr] = wv.y; sw[lk + 2][lr] = wv.z; sw[lk + 3][lr] = wv.w;
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; kk++) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; i++) { a[i] = sx[kk][ty * 4 + i]; b[i] = sw[kk][tx * 4 + i]; }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) acc[i][j] = fma(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int t = t0 + ty * 4 + i;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int e = e0 + tx * 4 + j;
            if (t < T && e < E) logits[(size_t)t * E + e] = acc[i][j];
        }
    }
}

int launch_router_logits_tiled(const float *x, int T, int H, const float *gate_w, int E, double *logits,
                               hipStream_t st)
{
    dim3 grid((T + 63) / 64, (E + 63) / 64);
    k_router_logits_tiled<<<grid, 256, 0, st>>>(x, T, H, gate_w, E, logits);
    return (int)hipGetLastError();
}

// one workgroup per token
__global__ __launch_bounds__(256) void k_topk(const RouteCfg rc, const double *__restrict__ logits,
                                              const float *__restrict__ bias, int T,
                                              int32_t *__restrict__ idx, float *__restrict__ w)
{
    __shared__ TopkLds tl;
    const int t = blockIdx.x;
    block_topk(rc, logits + (size_t)t * rc.E, bias, idx + (size_t)t * rc.k, w + (size_t)t * rc.k, tl);
}

int launch_topk(const RouteCfg &rc, const double *logits, const float *bias, int T, int32_t *idx,
                float *w, hipStream_t st)
{
    k_topk<<<T, 256, 0, st>>>(rc, logits, bias, T, idx, w);
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
