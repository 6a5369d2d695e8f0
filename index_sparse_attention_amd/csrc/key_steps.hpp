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
    int beg = 0;                                    // Q->K position of the row's first entry
    // optional per-entry values read along with the list (aux[i] for entry
    // i, i < aux_n; -1 past it): aux_at() gives the current entry's
    const int32_t* aux = nullptr;
    int aux_n = 0, achunk = -1;

    __device__ int kb_at() {
        if (list == nullptr) return it;
        const int base = it & ~63;
        if (base != chunk_base) {
            chunk_base = base;
            chunk = base + lane < count ? list[base + lane] : -1;
            if (aux != nullptr) achunk = base + lane < aux_n ? aux[base + lane] : -1;
        }
        return __builtin_amdgcn_readlane(chunk, it & 63);
    }
    __device__ int aux_at() const { return __builtin_amdgcn_readlane(achunk, it & 63); }
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

// The steps of query block qb of (batch b, query head h): the kept key blocks
// of its Q->K CSR row, or every key block of the sequence (dense), cut at
// the bottom-right causal diagonal of its last row.  a.Sq and a.Sk are the
// lengths of b's sequence; a.n_qb, a.n_kb the (longest) block counts the CSR
// rows are laid out with.
template <class Args>
__device__ __forceinline__ void init_key_steps(KeySteps& st, const Args& a, int b, int h, int qb, int lane) {
    st.lane = lane;
    st.n_kb = a.n_kb;
    const int last_row = min(qb * kBlock + kBlock - 1, a.Sq - 1);
    const int diag = last_row + a.Sk - a.Sq;
    st.last = a.causal ? min(diag, a.Sk - 1) : a.Sk - 1;
    if (a.mask_kind == 1) {
        const int hm = h * a.Hm / a.Hq;
        const int r = (b * a.Hm + hm) * a.n_qb + qb;
        const int beg = a.q2k_ptr[r];
        st.count = a.q2k_ptr[r + 1] - beg;
        st.list = a.q2k_col + beg;
        st.beg = beg;
    } else {
        const int nkb = (a.Sk + kBlock - 1) / kBlock;
        st.count = nkb;
        if (a.causal) st.count = diag < 0 ? 0 : min(nkb, diag / kBlock + 1);
    }
}

}  // namespace isattn
