// kd_handoff.h -- hand-off words between workgroups of one launch, gfx950.
//
// A producer workgroup publishes a unit of work in memory, a consumer on
// another compute unit waits for it (the fused backward's sweep and chunk
// workers; the few-heads forward's preparation workers and state passes).
#pragma once

#include <hip/hip_runtime.h>

namespace kd {

// Hand-off words between workgroups of one launch (a producer publishes a
// unit of work in memory, a consumer on another compute unit waits for it).
// A word carries the launch's epoch (words of earlier launches never match),
// the writer's XCD id and bit 0 = published; bit 1 = PUB_FLUSHED when the
// writer wrote its XCD's L2 back to memory before publishing, so that a
// reader on another XCD may read after an agent-scope acquire.
constexpr unsigned long long PUB_FLUSHED = 2ull;

__device__ __forceinline__ unsigned xcc_id() {
    return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11));   // HW_REG_XCC_ID[3:0]
}
__device__ __forceinline__ unsigned long long pub_word(unsigned epoch, unsigned xcc) {
    return ((unsigned long long)epoch << 32) | ((unsigned long long)(xcc & 0xffu) << 24) | 1ull;
}
// bounded wait of one thread for a flag of this launch that has the bits
// `need`; false when the bound ran out (then nothing may be read)
__device__ __forceinline__ bool pub_wait(const unsigned long long* fp, unsigned epoch, unsigned long long need,
                                         unsigned long long& w, unsigned spin) {
    for (unsigned s = 0; s < spin; ++s) {
        w = __hip_atomic_load(fp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((unsigned)(w >> 32) == epoch && (w & need) == need) return true;
        __builtin_amdgcn_s_sleep(2);
    }
    return false;
}

}  // namespace kd
