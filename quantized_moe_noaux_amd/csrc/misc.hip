// RMSNorm of the decode stack, the block-dot test export and the token
// permutation of the grouped path.
#include "moe_dev.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- rmsnorm
// out = x / sqrt(mean(x^2) + eps) * g, one workgroup per row; the sum of
// squares and the scaling in fp64 with a fixed reduction order.  A row is
// read once: every float4 of a thread is loaded before any arithmetic (a
// decode step normalises one 24 KB row, so load latency, not bandwidth, is
// what costs), kept in registers and reused for the output.
__global__ __launch_bounds__(256) void k_rmsnorm(const float *__restrict__ x, const float *__restrict__ g,
                                                 double eps, int H, float *out)
{
    __shared__ double red[4];
    const float *xr = x + (size_t)blockIdx.x * H;
    float *orow = out + (size_t)blockIdx.x * H;
    const int tid = threadIdx.x;
    const bool vec = (((uintptr_t)xr | (uintptr_t)g | (uintptr_t)orow) & 15) == 0;
    if (vec && (H & 3) == 0 && H <= 256 * 4 * kNormPer) {
        const int n4 = H / 4;
        float4 v[kNormPer];
        load_row_regs(xr, n4, v);
        const double r = row_rstd(v, H, eps, red);
#pragma unroll
        for (int j = 0; j < kNormPer; j++) {
            const int i = tid + 256 * j;
            if (i < n4)
                reinterpret_cast<float4 *>(orow)[i] = norm4(v[j], r, reinterpret_cast<const float4 *>(g)[i]);
        }
        return;
    }
    double ss = 0.0;
    for (int j = tid; j < H; j += 256) ss = fma((double)xr[j], (double)xr[j], ss);
    ss = wave_sum_d(ss);
    if (lane_id() == 0) red[wave_id()] = ss;
    __syncthreads();
    const double r = 1.0 / sqrt(((red[0] + red[1]) + (red[2] + red[3])) / H + eps);
    for (int j = tid; j < H; j += 256) orow[j] = (float)((double)xr[j] * r * (double)g[j]);
}

int launch_rmsnorm(const float *x, const float *g, double eps, int T, int H, float *out, hipStream_t st)
{
    k_rmsnorm<<<T, 256, 0, st>>>(x, g, eps, H, out);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------- block dots
// One thread per (token, row, 16-byte chunk): the same chunk arithmetic the
// expert kernels use, with the activation block sums formed on the fly.
template <int WB>
__global__ __launch_bounds__(256) void k_block_dots(const uint8_t *__restrict__ codes, int rows, int D,
                                                    const int8_t *__restrict__ q, int T, int32_t *__restrict__ out)
{
    const int cpr = D * WB / 128;  // chunks per row
    const long n = (long)T * rows * cpr;
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    if (gid >= n) return;
    const int c = (int)(gid % cpr);
    const long tr = gid / cpr;
    const int r = (int)(tr % rows), t = (int)(tr / rows);
    const uint4 w = *reinterpret_cast<const uint4 *>(codes + ((size_t)r * cpr + c) * 16);
    const int8_t *qt = q + (size_t)t * D;
    int32_t *o = out + ((size_t)t * rows + r) * (D / 32);
    if constexpr (WB == 8) {
        Act<8> A;
        const uint4 v = reinterpret_cast<const uint4 *>(qt)[c];
        A.a[0] = v.x; A.a[1] = v.y; A.a[2] = v.z; A.a[3] = v.w;
        A.d = 0.f;
        // two chunks make one block: the even chunk adds its partner's half
        if (c & 1) return;
        const uint4 w2 = *reinterpret_cast<const uint4 *>(codes + ((size_t)r * cpr + c + 1) * 16);
        Act<8> B;
        const uint4 v2 = reinterpret_cast<const uint4 *>(qt)[c + 1];
        B.a[0] = v2.x; B.a[1] = v2.y; B.a[2] = v2.z; B.a[3] = v2.w;
        B.d = 0.f;
        o[c >> 1] = A.isum(w) + B.isum(w2);
    } else if constexpr (WB == 4) {
        const uint4 *p = reinterpret_cast<const uint4 *>(qt + 32 * c);
        const uint4 v0 = p[0], v1 = p[1];
        uint32_t nn[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        Act<4> A;
        A.set(nn, 0.f);
        o[c] = A.isum(w);
    } else {
        const uint4 *p = reinterpret_cast<const uint4 *>(qt + 64 * c);
        uint32_t nn[16];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint4 v = p[i];
            nn[4 * i] = v.x; nn[4 * i + 1] = v.y; nn[4 * i + 2] = v.z; nn[4 * i + 3] = v.w;
        }
        Act<2> A;
        A.set(nn, 0.f, 0.f);
        int i0, i1;
        A.isum2(w, i0, i1);
        o[2 * c] = i0;
        o[2 * c + 1] = i1;
    }
}

// ---------------------------------------------------------------- streaming read (measurement aid)
// Thread i of the grid reads 16-byte chunks i, i + n, i + 2n, ... (n = the
// grid's thread count) eight at a time, so that a workgroup's load
// instruction covers one contiguous 4 KB window, with the non-temporal hint
// of the decode kernels' weight loads; the data only feeds an XOR.
constexpr int kStreamBlocks = 2048, kStreamThreads = 256, kStreamUnroll = 8;
__global__ __launch_bounds__(kStreamThreads) void k_stream_read(const uint4 *__restrict__ p, size_t n16,
                                                                uint32_t *__restrict__ sink)
{
    typedef unsigned v4u_s __attribute__((ext_vector_type(4)));
    const v4u_s *q = reinterpret_cast<const v4u_s *>(p);
    const size_t nthr = (size_t)kStreamBlocks * kStreamThreads;
    size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kStreamUnroll - 1) * nthr < n16; i += kStreamUnroll * nthr) {
        v4u_s v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; u++) v[u] = __builtin_nontemporal_load(q + i + u * nthr);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += nthr) {
        const v4u_s v = __builtin_nontemporal_load(q + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(size_t)blockIdx.x * kStreamThreads + threadIdx.x] = acc;
}

int launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t st)
{
    static_assert((size_t)kStreamBlocks * kStreamThreads == MOE_STREAM_SINK_WORDS, "sink size");
    k_stream_read<<<kStreamBlocks, kStreamThreads, 0, st>>>(static_cast<const uint4 *>(src), bytes / 16, sink);
    return (int)hipGetLastError();
}

int launch_block_dots(int wbits, const uint8_t *codes, int rows, int D, const int8_t *q, int T,
                      int32_t *out, hipStream_t st)
{
    const long n = (long)T * rows * (D * wbits / 128);
    const unsigned grid = (unsigned)((n + 255) / 256);
    if (wbits == 8) k_block_dots<8><<<grid, 256, 0, st>>>(codes, rows, D, q, T, out);
    else if (wbits == 4) k_block_dots<4><<<grid, 256, 0, st>>>(codes, rows, D, q, T, out);
    else k_block_dots<2><<<grid, 256, 0, st>>>(codes, rows, D, q, T, out);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------- permutation
// Stable counting sort of the T*k assignments by expert (batch-union MoE,
// GeekNews #31297 implemented features), in three launches:
//  k_perm_count  tile j of 256 assignments writes its per-expert counts
//  k_perm_scan   one block: per expert, the running sum over tiles (each
//                tile's start within its expert), then the exclusive scan
//                over experts gives off[]; optionally the grouped path's
//                tile list
//  k_perm_place  each assignment's row = off[e] + its tile's start + the
//                number of earlier assignments of the same expert in its tile
// An assignment of expert -1 (dropped by adaptive top-p) gets no row and
// inv = -1; the kept ones fill rows 0 .. off[E]-1.
__global__ __launch_bounds__(256) void k_perm_count(const int32_t *__restrict__ idx, int n, int E,
                                                    int32_t *__restrict__ cnt /*[tiles][E]*/)
{
    __shared__ int c[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += 256) c[e] = 0;
    __syncthreads();
    const int a = blockIdx.x * 256 + threadIdx.x;
    if (a < n) {
        const int e = idx[a];
        if (e >= 0 && e < E) atomicAdd(&c[e], 1);  // e = -1: dropped by top-p, no row
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) cnt[(size_t)blockIdx.x * E + e] = c[e];
}

// exclusive prefix sum over the 512 threads of a block (wave scans, then the
// eight wave totals); `tot` receives the block total
__device__ int block_scan_512(int v, int *wsum, int &tot)
{
    const int l = lane_id(), w = wave_id();
    int x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (l >= o) x += y;
    }
    if (l == kWave - 1) wsum[w] = x;
    __syncthreads();
    int pre = 0, all = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int s = wsum[i];
        pre += (i < w) ? s : 0;
        all += s;
    }
    tot = all;
    return pre + x - v;
}

__global__ __launch_bounds__(512) void k_perm_scan(int tiles, int E, int32_t *__restrict__ cnt,
                                                   int32_t *__restrict__ off, int4 *__restrict__ gtiles, int T,
                                                   int k, int n_shared)
{
    __shared__ int ws0[8], ws1[8];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        for (int j0 = 0; j0 < tiles; j0 += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; u++) v[u] = (j0 + u < tiles) ? cnt[(size_t)(j0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 8; u++)
                if (j0 + u < tiles) {
                    cnt[(size_t)(j0 + u) * E + e] = run;
                    run += v[u];
                }
        }
    }
    int total;
    const int base = block_scan_512(run, ws0, total);
    if (e < E) off[e] = base;
    if (e == 0) off[E] = total;
    if (!gtiles) return;
    const int nte = (e < E) ? (run + kGgTN - 1) / kGgTN : 0;
    int ntr;
    const int tb = block_scan_512(nte, ws1, ntr);
    for (int j = 0; j < nte; j++)
        gtiles[1 + tb + j] = make_int4(e, base + j * kGgTN, min(kGgTN, run - j * kGgTN), 0);
    const int Tk = T * k, ns = n_shared ? (T + kGgTN - 1) / kGgTN : 0;
    for (int j = e; j < ns; j += 512)
        gtiles[1 + ntr + j] = make_int4(E, Tk + j * kGgTN, min(kGgTN, T - j * kGgTN), 0);
    if (e == 0) gtiles[0] = make_int4(ntr + ns, 0, 0, 0);
}

__global__ __launch_bounds__(256) void k_perm_place(const int32_t *__restrict__ idx, int n, int E,
                                                    const int32_t *__restrict__ base,
                                                    const int32_t *__restrict__ off, int32_t *__restrict__ perm,
                                                    int32_t *__restrict__ inv)
{
    __shared__ int s_e[256];
    const int a0 = blockIdx.x * 256, a = a0 + threadIdx.x;
    s_e[threadIdx.x] = (a < n) ? idx[a] : -1;
    __syncthreads();
    if (a >= n) return;
    const int e = s_e[threadIdx.x];
    if (e < 0 || e >= E) {  // dropped by top-p: no row
        inv[a] = -1;
        return;
    }
    int r = 0;
    for (int j = 0; j < (int)threadIdx.x; j++) r += (s_e[j] == e);
    const int row = off[e] + base[(size_t)blockIdx.x * E + e] + r;
    perm[row] = a;
    inv[a] = row;
}

int launch_permute(const int32_t *idx, int T, int k, int E, int32_t *perm, int32_t *off, int32_t *inv,
                   int32_t *scratch, int4 *tiles, int n_shared, hipStream_t st)
{
    const int n = T * k, nt = perm_tiles(n);
    if (nt) k_perm_count<<<nt, 256, 0, st>>>(idx, n, E, scratch);
    k_perm_scan<<<1, 512, 0, st>>>(nt, E, scratch, off, tiles, T, k, n_shared);
    if (nt) k_perm_place<<<nt, 256, 0, st>>>(idx, n, E, scratch, off, perm, inv);
    return (int)hipGetLastError();
}

} // namespace moe
