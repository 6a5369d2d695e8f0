// Step sequence over the kept key blocks of one 128-row query block, shared by
// the kernels that stream K/V tiles past resident query rows (the SPLIT dQ
// pass, the forward).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bwd_args.hpp"

namespace isattn {

// Every 32-key part of every kept key block that holds a key some row of the
// query block sees (key <= last, the last key visible to the block's last
// row).  The kept key blocks are read 64 at a time into a register (one per
// lane).
struct KeySteps {
    int it = -1, sub = 0, count = 0, n0 = 0, n_kb = 0, last = 0, lane = 0;
    const int32_t* list = nullptr;
    int chunk = 0, chunk_base = -1;

    __device__ int kb_at() {
        if (list == nullptr) return it;
        const int base = it & ~63;
        if (base != chunk_base) {
            chunk_base = base;
            chunk = base + lane < count ? list[base + lane] : -1;
        }
        return __builtin_amdgcn_readlane(chunk, it & 63);
    }
    __device__ bool next_block() {
        for (;;) {
            if (++it >= count) return false;
            const int kb = kb_at();
            if (kb < 0 || kb >= n_kb) continue;     // malformed entry: nothing to do
            if (kb * kBlock > last) continue;
            sub = 0;
            n0 = kb * kBlock;
            return true;
        }
    }
    __device__ bool next() {
        if (++sub < kBlock / 32 && n0 + 32 <= last) {
            n0 += 32;
            return true;
        }
        return next_block();
    }
};

}  // namespace isattn
