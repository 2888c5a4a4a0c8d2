// Seeded synthetic inputs for the MoE layer: device side.
//
// Device twin of synth.c (same SplitMix64 definitions, integer-only apart
// from the exact-rounded fp64 multiply of the scales).  Used to fill the
// multi-gigabyte expert weight tensors directly in HBM; the host side can
// regenerate any single expert bit for bit.  No MoE arithmetic lives here.
//
// Stacked tensors: expert e of a stack lives at out + e * per_exp elements
// and is drawn from stream (stream_base | e).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

__device__ __forceinline__ uint64_t mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t key_of(uint64_t seed, uint64_t stream)
{
    return mix(mix(seed + kGamma) ^ stream);
}

__device__ __forceinline__ uint64_t word(uint64_t key, uint64_t i)
{
    return mix(key + (i + 1) * kGamma);
}

// one thread writes one 64-bit word = 8 raw bytes
__global__ void fill_bytes(uint64_t seed, uint64_t stream_base, uint64_t words_per_exp,
                           uint64_t total_words, uint64_t *out)
{
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t w = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total_words; w += stride) {
        uint64_t e = w / words_per_exp, i = w - e * words_per_exp;
        out[w] = word(key_of(seed, stream_base | e), i);
    }
}

// one thread writes 4 int8 codes from one word
__global__ void fill_int8(uint64_t seed, uint64_t stream_base, uint64_t words_per_exp,
                          uint64_t total_words, uint32_t *out)
{
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t w = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total_words; w += stride) {
        uint64_t e = w / words_per_exp, i = w - e * words_per_exp;
        uint64_t r = word(key_of(seed, stream_base | e), i);
        uint32_t packed = 0;
        for (int k = 0; k < 4; k++) {
            uint64_t v = (r >> (16 * k)) & 0xFFFFULL;
            int c = (int)((v * 255ULL) >> 16) - 127;
            packed |= ((uint32_t)(uint8_t)(int8_t)c) << (8 * k);
        }
        out[w] = packed;
    }
}

__global__ void fill_scales(uint64_t seed, uint64_t stream_base, uint64_t per_exp,
                            uint64_t total, double c, float *out)
{
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < total; j += stride) {
        uint64_t e = j / per_exp, i = j - e * per_exp;
        uint64_t u24 = word(key_of(seed, stream_base | e), i) >> 40;
        out[j] = (float)((0.5 + (double)u24 * 0x1p-24) * c);
    }
}

unsigned grid_for(uint64_t n)
{
    uint64_t g = (n + 255) / 256;
    return (unsigned)(g > 65536 ? 65536 : (g ? g : 1));
}

} // namespace

extern "C" {

// Fills n_exp * bytes_per_exp raw bytes; bytes_per_exp must be a multiple of 8
// and `out` 8-byte aligned.  Returns 0, or -1 on bad arguments, or the HIP error.
int synth_dev_bytes(uint64_t seed, uint64_t stream_base, int64_t n_exp, uint64_t bytes_per_exp,
                    void *out, hipStream_t stream)
{
    if (!out || n_exp < 0 || bytes_per_exp % 8 || ((uintptr_t)out & 7)) return -1;
    uint64_t wpe = bytes_per_exp / 8, total = wpe * (uint64_t)n_exp;
    if (!total) return 0;
    fill_bytes<<<grid_for(total), 256, 0, stream>>>(seed, stream_base, wpe, total, (uint64_t *)out);
    return (int)hipGetLastError();
}

// Fills n_exp * codes_per_exp int8 codes; codes_per_exp must be a multiple of 4.
int synth_dev_int8(uint64_t seed, uint64_t stream_base, int64_t n_exp, uint64_t codes_per_exp,
                   void *out, hipStream_t stream)
{
    if (!out || n_exp < 0 || codes_per_exp % 4 || ((uintptr_t)out & 3)) return -1;
    uint64_t wpe = codes_per_exp / 4, total = wpe * (uint64_t)n_exp;
    if (!total) return 0;
    fill_int8<<<grid_for(total), 256, 0, stream>>>(seed, stream_base, wpe, total, (uint32_t *)out);
    return (int)hipGetLastError();
}

// Fills n_exp * per_exp fp32 scales.
int synth_dev_scales(uint64_t seed, uint64_t stream_base, int64_t n_exp, uint64_t per_exp,
                     double c, float *out, hipStream_t stream)
{
    if (!out || n_exp < 0) return -1;
    uint64_t total = per_exp * (uint64_t)n_exp;
    if (!total) return 0;
    fill_scales<<<grid_for(total), 256, 0, stream>>>(seed, stream_base, per_exp, total, c, out);
    return (int)hipGetLastError();
}

} // extern "C"
