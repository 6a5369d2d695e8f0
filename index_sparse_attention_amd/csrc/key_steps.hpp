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
// row).  The kept key blocks are taken 64 list entries at a time, one per
// lane, tested lane-parallel and packed, so a step reads its block with one
// lane read.
struct KeySteps {
    int sub = 0, count = 0, n0 = 0, n_kb = 0, last = 0, lane = 0;
    const int32_t* list = nullptr;
    int beg = 0;                                    // Q->K position of the row's first entry
    // optional per-entry values read along with the list (aux[i] for entry
    // i, i < aux_n; -1 past it): aux_at() gives the current entry's
    const int32_t* aux = nullptr;
    int aux_n = 0;
    int scan = 0, pos = 0, nval = 0;                // next entry to take; current / number of packed
    int e_kb = 0, e_aux = -1;                       // packed entries, one per lane

    // take entries scan .. scan + 63: each lane tests its own (a valid block
    // index that holds a key some row sees) and the valid ones are packed to
    // the low lanes in list order
    __device__ void refill() {
        const int e = scan + lane;
        int kb = -1, x = -1;
        if (e < count) {
            kb = list != nullptr ? list[e] : e;
            if (aux != nullptr && e < aux_n) x = aux[e];
        }
        const bool v = kb >= 0 && kb < n_kb && kb * kBlock <= last;
        const uint64_t mask = __ballot(v);
        const int dst = v ? __popcll(mask & ((uint64_t(1) << lane) - 1)) : 63;
        e_kb = __builtin_amdgcn_ds_permute(dst * 4, kb);
        if (aux != nullptr) e_aux = __builtin_amdgcn_ds_permute(dst * 4, x);
        nval = __popcll(mask);
        pos = -1;
        scan += 64;
    }
    __device__ int aux_at() const { return __builtin_amdgcn_readlane(e_aux, pos); }
    __device__ bool next_block() {
        for (;;) {
            if (++pos < nval) {
                const int kb = __builtin_amdgcn_readlane(e_kb, pos);
                sub = 0;
                n0 = kb * kBlock;
                return true;
            }
            if (scan >= count) return false;
            refill();
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
