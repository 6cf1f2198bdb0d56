// Exhaustive host check of the selection's key map (key_map.h, the same
// header the kernels include) over all 2^32 float bit patterns:
//  - walking every non-NaN float in ascending value order (-inf, negative
//    normals and subnormals, -0, +0, positive subnormals and normals, +inf),
//    the float comparison agrees with the walk (so the walk is the value
//    order), and the key strictly increases at every step except -0 -> +0,
//    where it stays equal (the two zeros tie);
//  - key 0 ("no element") comes from no non-NaN pattern (it does come from
//    NaN patterns: 0xFFFFFFFF, and signalling NaNs that the +0.0 quiets to
//    it; NaN is outside the contract).
// Prints "ok <visited>" and exits 0, else prints the first failure and exits 1.
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "key_map.h"

static float as_float(uint32_t b) {
    float f;
    memcpy(&f, &b, sizeof(f));
    return f;
}

int main() {
    uint64_t visited = 0;
    bool have = false;
    float pf = 0.0f;
    uint32_t pk = 0, pb = 0;
    auto visit = [&](uint32_t b) -> bool {
        const float f = as_float(b);
        const uint32_t k = tks_key_of(f);
        if (have) {
            if (!(pf <= f)) {
                printf("walk not ascending at %08x -> %08x\n", pb, b);
                return false;
            }
            if (pf < f ? !(pk < k) : (pk != k)) {
                printf("key order broken: %08x (key %08x) -> %08x (key %08x)\n", pb, pk, b, k);
                return false;
            }
        }
        have = true;
        pf = f;
        pk = k;
        pb = b;
        ++visited;
        return true;
    };
    for (uint32_t b = 0xFF800000u; b > 0x80000000u; --b)
        if (!visit(b)) return 1;
    if (!visit(0x80000000u)) return 1;
    for (uint32_t b = 0u;; ++b) {
        if (!visit(b)) return 1;
        if (b == 0x7F800000u) break;
    }
    if (visited != 0x100000000ull - 0x1000000ull + 2u) {  // all but the 2^24 - 2 NaN patterns
        printf("visited %llu patterns\n", (unsigned long long)visited);
        return 1;
    }
    uint64_t zeros = 0;
    for (uint64_t b = 0; b <= 0xFFFFFFFFull; ++b) {
        if (tks_key_of(as_float((uint32_t)b)) != 0u) continue;
        const uint32_t mag = (uint32_t)b & 0x7FFFFFFFu;
        if (mag <= 0x7F800000u) {  // not a NaN
            printf("key 0 from the non-NaN pattern %08llx\n", (unsigned long long)b);
            return 1;
        }
        ++zeros;
    }
    if (tks_key_of(as_float(0xFFFFFFFFu)) != 0u || zeros == 0) {
        printf("the NaN pattern ffffffff does not map to 0\n");
        return 1;
    }
    printf("ok %llu\n", (unsigned long long)visited);
    return 0;
}
