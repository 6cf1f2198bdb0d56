// key_map.h - the mapping step of the radix select (the TopK article,
// section 02): float -> unsigned key, key(a) < key(b) iff a < b for non-NaN
// values.  Adding +0.0 turns -0.0 into +0.0 (IEEE round to nearest) and
// leaves every other value, subnormals included, unchanged, so -0.0 and +0.0
// get the same key and tie.  Negative values have all bits flipped,
// non-negative ones only the sign bit.  Key 0 marks "no element": no
// non-NaN value maps there (the NaN pattern 0xFFFFFFFF does, and signalling
// NaNs that the addition quiets to it; NaN is outside the contract).
//
// Plain C++ with no device intrinsics, compiled for the host and the GPU
// alike (the pragma makes it callable from kernels), so that a host program
// can check it over all 2^32 bit patterns.
#ifndef TOPK_SELECT_KEY_MAP_H_
#define TOPK_SELECT_KEY_MAP_H_

#include <stdint.h>
#include <string.h>

#pragma clang force_cuda_host_device begin

static inline uint32_t tks_key_of(float x) {
    x += 0.0f;
    uint32_t u;
    memcpy(&u, &x, sizeof(u));
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

#pragma clang force_cuda_host_device end

#endif  // TOPK_SELECT_KEY_MAP_H_
