// Host check of the one-token down kernel's slot record (slot_record.h):
// every field survives packing, including offsets below the base pointer.
#include <stdio.h>
#include <stdint.h>
#include "slot_record.h"

int main()
{
    const int64_t offs[] = {0, 16, (int64_t)1 << 33, ((int64_t)1 << 62) + 5, -16, -((int64_t)1 << 33),
                            -((int64_t)1 << 47) + 4096, INT64_MIN / 2, INT64_MAX / 3};
    const int pairs[] = {-1, 0, 1, 32, 263, moe::kRecordMaxPair};
    const int ws[] = {0, 0x3f800000, 0x40200000, (int)0x80000001};
    int bad = 0, n = 0;
    for (int64_t off : offs)
        for (int pair : pairs)
            for (int sh = 0; sh < 2; sh++)
                for (int wb : ws) {
                    moe::SlotRecord r;
                    r.off = off; r.pair = pair; r.shared = sh != 0; r.w_bits = wb;
                    int w[4];
                    moe::record_pack(r, w);
                    const moe::SlotRecord u = moe::record_unpack(w[0], w[1], w[2], w[3]);
                    n++;
                    if (u.off != off || u.pair != pair || u.shared != (sh != 0) || u.w_bits != wb) {
                        bad++;
                        printf("mismatch: off %lld pair %d shared %d w %d\n", (long long)off, pair, sh, wb);
                    }
                }
    printf("%d of %d records round-trip\n", n - bad, n);
    return bad ? 1 : 0;
}
