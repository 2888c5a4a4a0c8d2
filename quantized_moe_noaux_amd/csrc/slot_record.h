// The one-token down kernel's per-slot record (four 32-bit words in LDS):
//   w0, w1  the byte offset of the workgroup's rows from the routed or the
//           shared base pointer, signed (a tiered expert's rows may lie
//           below the routed base: the expert table's offsets are
//           differences of device addresses);
//   w2      the staged pair + 1 (0: the slot adds nothing) in bits 0-15,
//           bit 16 set for the shared expert;
//   w3      the pair's weight (fp32 bits).
// Packing and unpacking are plain integer code, so the CPU tests check them
// on the host.
#pragma once
#include <stdint.h>

namespace moe {

constexpr int kRecordMaxPair = 0xFFFE;  // largest staged pair index a record holds

struct SlotRecord {
    int64_t off;
    int pair;      // -1: none
    bool shared;
    int w_bits;
};

__host__ __device__ inline void record_pack(const SlotRecord &r, int (&w)[4])
{
    const uint64_t o = (uint64_t)r.off;
    w[0] = (int)(uint32_t)o;
    w[1] = (int)(uint32_t)(o >> 32);
    w[2] = (int)((uint32_t)(r.pair + 1) | (r.shared ? 0x10000u : 0u));
    w[3] = r.w_bits;
}

__host__ __device__ inline SlotRecord record_unpack(int w0, int w1, int w2, int w3)
{
    SlotRecord r;
    r.off = (int64_t)((uint64_t)(uint32_t)w1 << 32 | (uint32_t)w0);
    r.pair = (int)((uint32_t)w2 & 0xFFFFu) - 1;
    r.shared = ((uint32_t)w2 >> 16) != 0;
    r.w_bits = w3;
    return r;
}

} // namespace moe
