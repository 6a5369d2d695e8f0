// Work before the main passes of the backward, as device functions so that
// one launch can carry several of them (the SPLIT_DS set-up runs the work
// order, the dS position map and the delta rows as one kernel; LoopK and
// LoopQ run the delta rows in their own preprocess kernel).
#pragma once
#include "bwd_args.hpp"
#include "device_common.hpp"

namespace isattn {

// Delta rows: delta[b, h, i] = sum over d of dO[b,i,h,d] * O[b,i,h,d], the
// fp32 sum of exact bf16 products (it equals the row sum of P * dP, the
// term dS = P (dP - delta) subtracts; with NEG the row gets -delta, the value
// the two-pass dK/dV kernel starts its dP accumulators at), and where a.lse2 is set also
// lse2 = lse * log2(e); rows past a sequence's length get delta 0 and
// lse2 = +inf.  Rows are taken in (b, i, h) order, h fastest: the token-major
// memory order of O and dO, so a block reads whole token rows; they are
// written to the statistics arrays at (b, h, i).  Block `blk` of NT threads
// covers rows [blk * kPreRows * NT / L, ...) with L = DV / 8 lanes per row
// (8 bf16 each); every thread issues the 16-byte loads of its kPreRows rows
// (and their lse) before any arithmetic.
constexpr int kPreRows = 4;

template <int DV, int NT, bool NEG = false>
__device__ __forceinline__ void delta_rows(const BwdArgs& a, int64_t blk) {
    constexpr int L = DV / 8;
    constexpr int RPB = NT / L;        // rows per pass
    constexpr int R = kPreRows;
    static_assert(NT % L == 0 && L <= 64, "whole rows per wave");
    const int64_t rows = int64_t(a.B) * a.Hq * a.stat_ld;
    const int sub = threadIdx.x % L;
    int64_t row[R], stat[R];
    bool in[R];
    u32x4_t o[R], g[R];
    float l2[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        row[r] = (blk * R + r) * RPB + threadIdx.x / L;
        const int64_t h = row[r] % a.Hq;
        const int64_t bi = row[r] / a.Hq;
        const int64_t i = bi % a.stat_ld;
        const int64_t b = bi / a.stat_ld;
        stat[r] = (b * a.Hq + h) * a.stat_ld + i;
        o[r] = u32x4_t{0u, 0u, 0u, 0u};
        g[r] = u32x4_t{0u, 0u, 0u, 0u};
        l2[r] = __builtin_inff();
        in[r] = false;
        if (row[r] < rows) {
            // token row of (b, i): b * stride_b + i * stride_s, or for packed
            // sequences cu_q[b] + i (rows past the sequence's length are padding)
            int64_t ob = b * a.o_sb + i * a.o_ss, db = b * a.do_sb + i * a.do_ss;
            int sq = a.Sq;
            if (a.cu_q != nullptr) {
                const int64_t t = a.cu_q[b] + i;
                sq = seq_len(a.cu_q, int(b), a.Sq);
                ob = t * a.o_ss;
                db = t * a.do_ss;
            }
            in[r] = i < sq;
            if (in[r]) {
                // read once: non-temporal, so they do not displace cached lines
                o[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.o + ob + h * a.o_sh + 8 * sub));
                g[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.dO + db + h * a.do_sh + 8 * sub));
                if (a.lse2 != nullptr) l2[r] = a.lse[(b * a.Hq + h) * a.lse_ld + i] * kLog2e;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc = fmaf(bf16_lo(o[r][j]), bf16_lo(g[r][j]), acc);
            acc = fmaf(bf16_hi(o[r][j]), bf16_hi(g[r][j]), acc);
        }
#pragma unroll
        for (int m = L / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, 64);
        if (row[r] < rows && sub == 0) {
            a.delta[stat[r]] = NEG ? -acc : acc;
            if (a.lse2 != nullptr) a.lse2[stat[r]] = l2[r];
        }
    }
}

template <int DV, int NT>
__host__ __device__ constexpr int delta_rows_per_block() {
    return kPreRows * (NT / (DV / 8));
}

// dS position map of SPLIT_DS with a block CSR: the K->Q position of every
// Q->K entry (the slot of the dS tile the dK/dV pass stores for that block),
// one wave per Q->K row (b, hm, qb), lanes over its entries, each a binary
// search for qb in the K->Q row (b, hm, kb); -1 where the two forms
// disagree.  Block `blk` of NT threads covers rows blk * NT/64 ... .  Thread
// 0 of block 0 also sets the overflow flag: the CSR holds more blocks than
// the map or the dS tiles have room for.
template <int NT>
__device__ __forceinline__ void ds_map_rows(const BwdArgs& a, int64_t blk) {
    if (blk == 0 && threadIdx.x == 0) {
        const int64_t rq = int64_t(a.B) * a.Hm * a.n_qb, rk = int64_t(a.B) * a.Hm * a.n_kb;
        const int64_t nnz = max(int64_t(a.q2k_ptr[rq]), int64_t(a.k2q_ptr[rk]));
        *a.ds_flag = (nnz > a.ds_map_len || nnz * (a.Hq / a.Hm) > a.ds_cap) ? 1 : 0;
    }
    const int64_t row = blk * (NT / 64) + (threadIdx.x >> 6);
    if (row >= int64_t(a.B) * a.Hm * a.n_qb) return;
    const int lane = threadIdx.x & 63;
    const int64_t bhm = row / a.n_qb;
    const int qb = int(row - bhm * a.n_qb);
    const int end = a.q2k_ptr[row + 1];
    for (int p = a.q2k_ptr[row] + lane; p < end; p += 64) {
        if (p < 0 || p >= a.ds_map_len) continue;
        const int kb = a.q2k_col[p];
        int pos = -1;
        if (kb >= 0 && kb < a.n_kb) {
            const int64_t r = bhm * a.n_kb + kb;
            const int hi0 = a.k2q_ptr[r + 1];
            int lo = a.k2q_ptr[r], hi = hi0;
            while (lo < hi) {
                const int mid = lo + (hi - lo) / 2;
                if (a.k2q_col[mid] < qb) lo = mid + 1;
                else hi = mid;
            }
            if (lo < hi0 && a.k2q_col[lo] == qb) pos = lo;
        }
        a.ds_map[p] = pos;
    }
}

}  // namespace isattn
