// Atomic-free attention backward: two passes that each keep their outputs on
// chip and store them once, recomputing P and dS in both.
//
// The loop orders are the two of MagiAttention PR #334 (Summary): the
// Q-outer pass is LoopK restricted to dQ, the K-outer pass is LoopQ restricted
// to dK/dV.  On MI355X fp32 global atomics run at about a quarter of the
// plain-store rate, so reducing dK/dV (LoopK) or dQ (LoopQ) through them
// bounds the fused kernels far below the MFMA peak; spending 1.4x the MFMA
// work on a second S/dP recompute removes every atomic and the fp32
// workspace.
//
// dQ pass (k_bwd_dq): workgroup = one 128-row query tile; each wave owns WR
// query rows with their Q / dO rows resident in registers.  Per 32-key step:
// S^T = K Q^T and dP^T = V dO^T (A = K/V from LDS), P and dS in registers,
// dQ += dS K with dS taken straight from the accumulators and K read back with
// transposing LDS loads.  K/V rows are staged at LDS row swap23(r), which makes
// each lane's accumulator registers cover 8 consecutive keys.  This pass runs
// first: its prologue also computes each query row's delta = rowsum(dO * O)
// and lse * log2(e) and stores them for the dK/dV pass, so the backward needs
// no separate preprocess launch.
//
// dK/dV pass (k_bwd_dkdv): workgroup = one 128-key tile, eight waves in two
// roles (P waves with K resident and dV accumulators, dS waves with V resident
// and dK accumulators) exchanging P through LDS; the Q/dO tiles of each query
// step are staged once and read by both roles.
//
// Both passes fill their LDS rings with direct global->LDS loads issued from
// inside the MFMA stream, a step or two ahead, and take one workgroup barrier
// per step.
#include <climits>
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "key_steps.hpp"
#include "pre_rows.hpp"

namespace isattn {
namespace {

// ---------------------------------------------------------------------------
// Work order
//
// Each pass's work items are cut into 8 contiguous ranges -- the ranges
// xcd_item hands to the 8 XCDs, so an XCD's workgroups share operand tiles in
// its L2 -- and each range is sorted by decreasing work (the kept blocks the
// item visits): every XCD starts its longest items first and the shortest
// fill the end (longest-processing-time-first list scheduling).  Counting
// sort on min(work, kSchedKeys - 1); items of equal work land in any order,
// which never changes a result (every item writes only its own outputs).
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;
constexpr int kSchedKeys = 4096;

// kept query blocks a dK/dV item (b, KV head, key block) visits, over its GQA group
__device__ int item_work_kv(const BwdArgs& a0, int item) {
    BwdArgs a = a0;
    const int bh = item / a.n_kb;
    const int kb = item - bh * a.n_kb;
    const int b = bh / a.Hk;
    const int hk = bh - b * a.Hk;
    if (a.cu_q != nullptr) seq_view(a, b);
    if (kb * kBlock >= a.Sk) return 0;             // past the end of b's keys
    if (a.mask_kind == 1) {
        int w = 0;
        for (int g = 0; g < a.G; ++g) {
            const int h = hk * a.G + g;
            const int r = (b * a.Hm + h * a.Hm / a.Hq) * a.n_kb + kb;
            w += a.k2q_ptr[r + 1] - a.k2q_ptr[r];
        }
        return w;
    }
    const int first_row = kb * kBlock - (a.Sk - a.Sq);
    const int first = a.causal && first_row > 0 ? first_row / kBlock : 0;
    return a.G * max(0, (a.Sq + kBlock - 1) / kBlock - first);
}
// kept key blocks a dQ item (b, query head, query block) visits
__device__ int item_work_q(const BwdArgs& a0, int item) {
    BwdArgs a = a0;
    const int bh = item / a.n_qb;
    const int qb = item - bh * a.n_qb;
    const int b = bh / a.Hq;
    const int h = bh - b * a.Hq;
    if (a.cu_q != nullptr) seq_view(a, b);
    if (qb * kBlock >= a.Sq) return 0;             // past the end of b's queries
    if (a.mask_kind == 1) {
        const int r = (b * a.Hm + h * a.Hm / a.Hq) * a.n_qb + qb;
        return a.q2k_ptr[r + 1] - a.q2k_ptr[r];
    }
    const int nkb = (a.Sk + kBlock - 1) / kBlock;
    if (!a.causal) return nkb;
    const int diag = min(qb * kBlock + kBlock - 1, a.Sq - 1) + (a.Sk - a.Sq);
    return diag < 0 ? 0 : min(nkb, diag / kBlock + 1);
}

// Exclusive block-wide scan of one value per thread (kSchedThreads threads);
// returns this thread's prefix, *total gets the sum.
__device__ int block_scan(int v, int* wsum, int* total) {
    const int tid = threadIdx.x, lane = tid & 63;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[tid >> 6] = incl;
    __syncthreads();
    int pre = incl - v, tot = 0;
    for (int w = 0; w < kSchedThreads / 64; ++w) {
        if (w < (tid >> 6)) pre += wsum[w];
        tot += wsum[w];
    }
    __syncthreads();
    *total = tot;
    return pre;
}

// Part mode of the dK/dV pass (fewer than kPartModeItems items, so at most
// one item per thread): item i gets P_i = ceil(work_i / T) parts (at most
// kMaxParts), the units (i, p) are sorted by decreasing part length into
// a.units (count at a.units[kv_units_bound]), and items with P_i > 1 get
// consecutive fp32 partial slots.
__device__ void schedule_parts(const BwdArgs& a, int* cnt, int* wsum) {
    const int n = a.B * a.Hk * a.n_kb;
    const int tid = threadIdx.x;
    int work = 0, parts = 0, len = 0;
    if (tid < n) {
        work = item_work_kv(a, tid);
        parts = min(kMaxParts, max(1, (work + a.kv_parts_T - 1) / a.kv_parts_T));
        len = (work + parts - 1) / parts;
    }
    int n_units = 0, n_slots = 0;
    block_scan(parts, wsum, &n_units);
    const int slot = block_scan(parts > 1 ? parts : 0, wsum, &n_slots);
    if (tid < n) {
        a.item_info[3 * tid] = work;
        a.item_info[3 * tid + 1] = parts;
        a.item_info[3 * tid + 2] = slot;
    }
    if (tid == 0) a.units[a.kv_units_bound] = n_units;
    const int key = kSchedKeys - 1 - min(len, kSchedKeys - 1);
    for (int k = tid; k < kSchedKeys; k += kSchedThreads) cnt[k] = 0;
    __syncthreads();
    if (tid < n) atomicAdd(&cnt[key], parts);
    __syncthreads();
    constexpr int PER = kSchedKeys / kSchedThreads;
    int v[PER];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        v[j] = cnt[PER * tid + j];
        sum += v[j];
    }
    int total = 0;
    int run = block_scan(sum, wsum, &total);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        cnt[PER * tid + j] = run;
        run += v[j];
    }
    __syncthreads();
    if (tid < n) {
        const int at = atomicAdd(&cnt[key], parts);
        for (int q = 0; q < parts; ++q) a.units[at + q] = (tid << 6) | q;
    }
}

// workgroup blk = (pass, XCD range): counting sort of the range into a.order
__device__ __forceinline__ void schedule_range(const BwdArgs& a, int blk, int* cnt, int* wsum, int* s_total_p) {
    const int pass = blk / kXcds;
    const int x = blk - pass * kXcds;
    if (pass == 0 && a.kv_parts_T > 0) {            // part mode: one workgroup schedules the dK/dV units
        if (x == 0) schedule_parts(a, cnt, wsum);
        return;
    }
    const int n_kv = a.B * a.Hk * a.n_kb;
    const int n = pass == 0 ? n_kv : a.B * a.Hq * a.n_qb;
    int32_t* out = a.order + (pass == 0 ? 0 : n_kv);
    const int per = xcd_items_per(n);
    const int lo = min(n, x * per);
    const int hi = min(n, lo + per);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // dK/dV items with at least 8 per CU of the XCD: grouped by (batch, KV
    // head), longest first inside a group, so the workgroups an XCD runs at
    // once share one head's Q and dO rows in its L2 (with fewer items per CU
    // the late start of a group's longest items would lengthen the tail).
    // Items with more than twice the range's mean work still go first, ahead
    // of every group, for the same reason.
    const int wmax = a.G * a.n_qb;
    const int ngrp = (hi - lo + a.n_kb - 1) / a.n_kb + 1;
    const bool grouped = pass == 0 && hi - lo >= 8 * kCusPerXcd && int64_t(ngrp + 1) * (wmax + 1) <= kSchedKeys;
    // the work of a thread's first kCache items, computed once
    constexpr int kCache = 4;
    auto work_of = [&](int i) { return pass == 0 ? item_work_kv(a, i) : item_work_q(a, i); };
    int wc[kCache];
#pragma unroll
    for (int j = 0; j < kCache; ++j) {
        const int i = lo + tid + j * kSchedThreads;
        wc[j] = i < hi ? work_of(i) : 0;
    }
    const int i_rest = lo + tid + kCache * kSchedThreads;
    int& s_total = *s_total_p;
    for (int k = tid; k < kSchedKeys; k += kSchedThreads) cnt[k] = 0;
    if (tid == 0) s_total = 0;
    __syncthreads();
    int big = INT_MAX;
    if (grouped) {
        int part = 0;
#pragma unroll
        for (int j = 0; j < kCache; ++j) part += wc[j];
        for (int i = i_rest; i < hi; i += kSchedThreads) part += work_of(i);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
        if (lane == 0) atomicAdd(&s_total, part);   // one LDS atomic per wave
        __syncthreads();
        big = int(2.f * float(s_total) / float(hi - lo));
    }
    auto key = [&](int i, int wk) {
        if (grouped) {
            const int lead = wmax - min(wk, wmax);
            return wk > big ? lead : (1 + i / a.n_kb - lo / a.n_kb) * (wmax + 1) + lead;
        }
        return kSchedKeys - 1 - min(wk, kSchedKeys - 1);
    };
#pragma unroll
    for (int j = 0; j < kCache; ++j) {
        const int i = lo + tid + j * kSchedThreads;
        if (i < hi) atomicAdd(&cnt[key(i, wc[j])], 1);
    }
    for (int i = i_rest; i < hi; i += kSchedThreads) atomicAdd(&cnt[key(i, work_of(i))], 1);
    __syncthreads();
    // exclusive scan of the counts: thread t owns keys PER * t .. PER * t + PER - 1
    constexpr int PER = kSchedKeys / kSchedThreads;
    int v[PER];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        v[j] = cnt[PER * tid + j];
        sum += v[j];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[tid >> 6] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < (tid >> 6); ++w) run += wsum[w];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        cnt[PER * tid + j] = run;
        run += v[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kCache; ++j) {
        const int i = lo + tid + j * kSchedThreads;
        if (i < hi) out[lo + atomicAdd(&cnt[key(i, wc[j])], 1)] = i;
    }
    for (int i = i_rest; i < hi; i += kSchedThreads) out[lo + atomicAdd(&cnt[key(i, work_of(i))], 1)] = i;
}

// Set-up of the two-pass backward, one launch: workgroups [0, n_sched) sort
// the work order (schedule_range), the next n_map build the dS position map
// of SPLIT_DS with a block CSR, the rest compute the delta and lse2 rows of
// SPLIT_DS (DV = 0: none).  The three read disjoint inputs and write disjoint
// outputs, so they run side by side; the passes that use them start after
// this kernel ends.
template <int DV>
__global__ __launch_bounds__(kSchedThreads) void k_split_setup(BwdArgs a, int32_t n_sched, int32_t n_map) {
    __shared__ int cnt[kSchedKeys];
    __shared__ int wsum[kSchedThreads / 64];
    __shared__ int s_total;
    const int blk = blockIdx.x;
    if (blk < n_sched) {
        schedule_range(a, blk, cnt, wsum, &s_total);
    } else if (blk < n_sched + n_map) {
        ds_map_rows<kSchedThreads>(a, blk - n_sched);
    } else if constexpr (DV > 0) {
        delta_rows<DV, kSchedThreads, true>(a, blk - n_sched - n_map);
    }
}

// ---------------------------------------------------------------------------
// dQ pass
//
// One workgroup per (batch, query head, 128-row query block); each wave owns
// WR rows: their Q and dO rows stay in registers (B operands), dQ in
// accumulators.  A step is 32 keys of a kept key block: S = K Q^T and
// dP = V dO^T from the K/V tile in LDS, then P, dS = P (dP - delta), and the
// dQ += dS K MFMAs of that step run at the start of the next one.  K/V tiles
// go through a 4-stage LDS ring filled by direct global->LDS loads issued two
// steps ahead from inside the MFMA stream.
// ---------------------------------------------------------------------------
template <int DQK, int DV, int WR, bool TOK>
struct DqCfg {
    static constexpr int BM = 128;                 // query rows per workgroup
    static constexpr int BN = 32;                  // keys per step
    static constexpr int NW = BM / WR;
    static constexpr int NT = 64 * NW;
    static constexpr int QT = WR / 32;             // 32-row query tiles per wave
    static constexpr int K_BYTES = BN * DQK * 2;
    static constexpr int V_BYTES = BN * DV * 2;
    static constexpr int TILE_BYTES = K_BYTES + V_BYTES;
    // token-exact masks: each wave's rows' bit words of the step (64 lanes x 4 B)
    static constexpr int TK_BYTES = TOK ? NW * 256 : 0;
    static constexpr int STAGE_BYTES = TILE_BYTES + TK_BYTES;
    static constexpr int NS = 4;                   // LDS ring stages (loads run two steps ahead)
    static constexpr int LDS_BYTES = NS * STAGE_BYTES;
    static constexpr int NKI = K_BYTES / 1024;     // 1 KiB loads per K tile
    static constexpr int NI = TILE_BYTES / 1024;   // 1 KiB loads per step
    static constexpr int KMAX = NI / NW;           // tile loads per wave per step
    static constexpr int NL = KMAX + (TOK ? 1 : 0);   // loads per wave per step
    static constexpr int NCQ = DQK / 16;
    static constexpr int NCV = DV / 16;
    static constexpr int NDT = DQK / 32;
    static_assert(NI % NW == 0 && K_BYTES % 1024 == 0, "tiles split into whole wave loads");
    static_assert(NL <= NCQ, "loads must fit between the S MFMAs");
    static_assert(!TOK || QT == 1, "token words: one query row per lane");
};

template <int DQK, int DV, int WR, bool VL, bool TOK>
// two workgroups per CU (two waves per SIMD) where the registers allow
__global__ __launch_bounds__(64 * (128 / WR), DQK > 128 ? 1 : 2) void k_bwd_dq(BwdArgs a) {
    using C = DqCfg<DQK, DV, WR, TOK>;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h2 = lane >> 5;

    // items (b, h, query block) in the per-XCD work order
    const int slot = xcd_item(blockIdx.x, a.n_qb * a.B * a.Hq);
    if (slot < 0) return;
    const int item = a.order[a.B * a.Hk * a.n_kb + slot];
    const int bh = item / a.n_qb;
    const int qb = item - bh * a.n_qb;
    const int b = bh / a.Hq;
    const int h = bh - b * a.Hq;
    const int hk = h / a.G;
    const int m_base = qb * C::BM;
    if constexpr (VL) {                            // packed sequences: narrow to sequence b
        seq_view(a, b);
        if (m_base >= a.Sq) return;                // a block past the end of the sequence
    }
    const int shift = a.Sk - a.Sq;

    KeySteps steps;
    init_key_steps(steps, a, b, h, qb, lane);

    // ---- resident operands: this wave's Q / dO rows (B operands), and the
    // rows' statistics, computed here and stored for the dK/dV pass (which
    // runs after this one): delta = rowsum(dO * O) over the lane's half of the
    // O row at the same positions as its dO operands plus the partner lane's
    // half (stored as -delta), and lse2 = lse * log2(e).  Padding rows past
    // Sq get lse2 = +inf (P = 0) and delta = 0.
    const int wrow = w * WR;
    bf16x8_t qB[C::QT][C::NCQ], doB[C::QT][C::NCV];
    float lse2[C::QT], dlt[C::QT];
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt) {
        const int qrow = m_base + wrow + 32 * qt + l32;
        const bool in = qrow < a.Sq;
        const uint16_t* qr = a.q + b * a.q_sb + h * a.q_sh + int64_t(in ? qrow : 0) * a.q_ss + 8 * h2;
        const uint16_t* dr = a.dO + b * a.do_sb + h * a.do_sh + int64_t(in ? qrow : 0) * a.do_ss + 8 * h2;
        const uint16_t* orow = a.o + b * a.o_sb + h * a.o_sh + int64_t(in ? qrow : 0) * a.o_ss + 8 * h2;
#pragma unroll
        for (int c = 0; c < C::NCQ; ++c) qB[qt][c] = in ? gload_operand(qr + 16 * c) : bf16x8_t{};
        u32x4_t ov[C::NCV];
#pragma unroll
        for (int c = 0; c < C::NCV; ++c) {
            doB[qt][c] = in ? gload_operand(dr + 16 * c) : bf16x8_t{};
            ov[c] = in ? gload128(orow + 16 * c) : u32x4_t{0u, 0u, 0u, 0u};
        }
        lse2[qt] = in ? a.lse[(int64_t(b) * a.Hq + h) * a.lse_ld + qrow] * kLog2e : __builtin_inff();
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < C::NCV; ++c) {
            const u32x4_t g = __builtin_bit_cast(u32x4_t, doB[qt][c]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc = fmaf(bf16_lo(ov[c][j]), bf16_lo(g[j]), acc);
                acc = fmaf(bf16_hi(ov[c][j]), bf16_hi(g[j]), acc);
            }
        }
        dlt[qt] = acc + __shfl_xor(acc, 32, 64);
        if (h2 == 0) {
            const int64_t si = (int64_t(b) * a.Hq + h) * a.stat_ld + qrow;
            a.lse2[si] = lse2[qt];
            a.delta[si] = -dlt[qt];             // negated: the dK/dV pass starts dP there
        }
    }

    f32x16_t dq[C::QT][C::NDT];
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
        for (int t = 0; t < C::NDT; ++t) dq[qt][t] = f32x16_t{};

    // ---- K/V tile loads: per-lane byte offsets of this wave's 1 KiB loads
    // (load k is instruction j = w + NW * k of the step: K tile parts, then V)
    const uint16_t* gk = a.k + b * a.k_sb + hk * a.k_sh;
    const uint16_t* gv = a.v + b * a.v_sb + hk * a.v_sh;
    const uint32_t lds_base = lds_address(lds);
    auto tile_off = [&](int j, int lim) -> uint32_t {      // tile rows past lim read row lim
        const bool is_k = j < C::NKI;
        const int jj = is_k ? j : j - C::NKI;
        const int D = is_k ? DQK : DV;
        const int e = 512 * jj + 8 * lane;
        const int r = e / D;
        const int c = ((e - r * D) >> 3) ^ chunk_swz(r, D);
        return uint32_t(min(swap23(r), lim)) * uint32_t((is_k ? a.k_ss : a.v_ss) * 2) + uint32_t(16 * c);
    };
    uint32_t toff[C::KMAX];
#pragma unroll
    for (int k = 0; k < C::KMAX; ++k) toff[k] = tile_off(w + C::NW * k, C::BN);
    struct Dma {
        uint32_t sb;
        uint32_t off[C::KMAX];
        const uint32_t* tk;                        // token words of the step's key group (TOK)
    } d;
    // token-exact bits: slot (b, mask head, qb, kb) row-major words; lane L
    // loads its row's word (row wrow + L % 32) for the step's 32 keys
    const uint32_t* tslots = nullptr;
    const uint32_t tk_off = uint32_t(16 * (w * WR + l32));
    if constexpr (TOK) tslots = a.tok + ((int64_t(b) * a.Hm + h * a.Hm / a.Hq) * a.n_qb + qb) * int64_t(a.n_kb) * 1024;
    auto plan = [&](int n0, int s) {
        d.sb = lds_base + uint32_t(s * C::STAGE_BYTES);
        if constexpr (TOK) d.tk = tslots + int64_t(n0 / kBlock) * 1024 + (n0 % kBlock) / 32;
        if (n0 + C::BN <= a.Sk) {
            const uint32_t mk = uint32_t(n0) * uint32_t(a.k_ss * 2), mv = uint32_t(n0) * uint32_t(a.v_ss * 2);
#pragma unroll
            for (int k = 0; k < C::KMAX; ++k) d.off[k] = toff[k] + (w + C::NW * k < C::NKI ? mk : mv);
        } else {                                   // ragged tail: keys past Sk re-read key Sk - 1
            const int nb = min(n0, a.Sk - 1);
            const uint32_t mk = uint32_t(nb) * uint32_t(a.k_ss * 2), mv = uint32_t(nb) * uint32_t(a.v_ss * 2);
#pragma unroll
            for (int k = 0; k < C::KMAX; ++k)
                d.off[k] = tile_off(w + C::NW * k, a.Sk - 1 - nb) + (w + C::NW * k < C::NKI ? mk : mv);
        }
    };
    auto restage = [&](int s) { d.sb = lds_base + uint32_t(s * C::STAGE_BYTES); };
    auto fire = [&](int k) {
        if (TOK && k == C::KMAX) {                 // this wave's rows' token words
            dma4(d.tk, tk_off, d.sb + uint32_t(C::TILE_BYTES + 256 * w));
            return;
        }
        const int j = w + C::NW * k;
        const bool is_k = j < C::NKI;
        dma16(is_k ? static_cast<const void*>(gk) : static_cast<const void*>(gv), d.off[k],
              d.sb + uint32_t(is_k ? 1024 * j : C::K_BYTES + 1024 * (j - C::NKI)));
    };

    // K^T fragment f = (cc, dt) of the dQ MFMAs from stage sp
    auto k_frag = [&](int sp, int f) {
        return b_operand_tr_swz<DQK>(lds + sp * (C::STAGE_BYTES / 2), 0, f / C::NDT, 32 * (f % C::NDT), lane);
    };
    // S and dP MFMAs of the step in stage s; the loads for two steps ahead go
    // out between them
    auto sdp = [&](int s, f32x16_t (&st)[C::QT], f32x16_t (&dpt)[C::QT]) {
        const uint16_t* sK = lds + s * (C::STAGE_BYTES / 2);
        const uint16_t* sV = sK + C::K_BYTES / 2;
#pragma unroll
        for (int qt = 0; qt < C::QT; ++qt) {
            st[qt] = f32x16_t{};
            dpt[qt] = f32x16_t{};
        }
        constexpr int PF = 2;                      // prefetch depth (chunks)
        bf16x8_t ka[PF + 1], va[PF + 1];
#pragma unroll
        for (int c = 0; c < PF; ++c) {
            ka[c] = row_operand_swz<DQK>(sK, l32, 16 * c + 8 * h2);
            if (c < C::NCV) va[c] = row_operand_swz<DV>(sV, l32, 16 * c + 8 * h2);
        }
#pragma unroll
        for (int c = 0; c < C::NCQ; ++c) {
            if (c + PF < C::NCQ) ka[(c + PF) % (PF + 1)] = row_operand_swz<DQK>(sK, l32, 16 * (c + PF) + 8 * h2);
            if (c + PF < C::NCV) va[(c + PF) % (PF + 1)] = row_operand_swz<DV>(sV, l32, 16 * (c + PF) + 8 * h2);
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt) st[qt] = mfma32(ka[c % (PF + 1)], qB[qt][c], st[qt]);
            if (c < C::NCV) {
#pragma unroll
                for (int qt = 0; qt < C::QT; ++qt) dpt[qt] = mfma32(va[c % (PF + 1)], doB[qt][c], dpt[qt]);
            }
            if (c < C::NL) fire(c);
        }
    };
    // this wave's token word of the step in stage s (TOK)
    auto tok_word = [&](int s) -> uint32_t {
        if constexpr (TOK)
            return *reinterpret_cast<const uint32_t*>(lds + (s * C::STAGE_BYTES + C::TILE_BYTES + 256 * w + 4 * l32) / 2);
        return ~0u;
    };
    // P and dS of a step (packed into dsn, accumulator register i holding key
    // n0 + 16*(i/8) + 8*h2 + i%8) with, when PREV, the dQ += dS K MFMAs of the
    // previous step (its dS in dsp, its K in stage sp) issued between the
    // arithmetic.  Masked steps clear the packed pairs afterwards.
    bf16x8_t dsp[C::QT][2];
    auto ds_step = [&](auto prev, int sp, const f32x16_t (&st)[C::QT], const f32x16_t (&dpt)[C::QT], int n0,
                       bf16x8_t (&dsn)[C::QT][2], uint32_t tw) {
        constexpr bool PREV = decltype(prev)::value;
        constexpr int NF = 2 * C::NDT;             // dQ B fragments, f = cc * NDT + dt
        constexpr int PF = NF < 3 ? NF : 3;        // prefetch depth
        constexpr int NP = 8 * C::QT;              // packed pairs (qt, cc, jj)
        bf16x8_t fr[PF + 1];
        if (PREV) {
#pragma unroll
            for (int f = 0; f < PF; ++f) fr[f] = k_frag(sp, f);
        }
        u32x4_t pk[C::QT][2];
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (PREV) {
                if (f + PF < NF) fr[(f + PF) % (PF + 1)] = k_frag(sp, f + PF);
                const int cc = f / C::NDT, dt = f % C::NDT;
#pragma unroll
                for (int qt = 0; qt < C::QT; ++qt) dq[qt][dt] = mfma32(dsp[qt][cc], fr[f % (PF + 1)], dq[qt][dt]);
            }
#pragma unroll
            for (int q = f * NP / NF; q < (f + 1) * NP / NF; ++q) {
                const int qt = q >> 3, cc = (q >> 2) & 1, jj = q & 3;
                float r[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int i = 8 * cc + 2 * jj + e;
                    const float pv = fast_exp2(st[qt][i] * a.scale_log2 - lse2[qt]);
                    r[e] = pv * (dpt[qt][i] - dlt[qt]);
                }
                pk[qt][cc][jj] = pack_bf16x2(r[0], r[1]);
            }
            __builtin_amdgcn_sched_barrier(0);     // keep one MFMA and its share of the arithmetic together
        }
        if ((n0 + C::BN > a.Sk) || (a.causal && n0 + C::BN - 1 > m_base + shift)) {
            // keys past Sk or (causal) past the row's last visible key: clear the pair halves
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt) {
                const int qrow = m_base + wrow + 32 * qt + l32;
                const int rel = min(a.Sk - 1, a.causal ? qrow + shift : a.Sk - 1) - n0 - 8 * h2;
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int o = 16 * cc + 2 * jj;
                        pk[qt][cc][jj] &= (o <= rel ? 0x0000ffffu : 0u) | (o + 1 <= rel ? 0xffff0000u : 0u);
                    }
            }
        }
        if constexpr (TOK) {                       // keys the row did not select
            const uint32_t mine = tw >> (8 * h2);
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int o = 16 * cc + 2 * jj;
                    pk[0][cc][jj] &= (((mine >> o) & 1u) ? 0x0000ffffu : 0u) | (((mine >> (o + 1)) & 1u) ? 0xffff0000u : 0u);
                }
        }
#pragma unroll
        for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) dsn[qt][cc] = as_bf16x8(pk[qt][cc]);
    };
    // dQ += dS K of the last step (stage sp)
    auto dq_last = [&](int sp) {
        constexpr int NF = 2 * C::NDT;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const bf16x8_t fr = k_frag(sp, f);
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt) dq[qt][f % C::NDT] = mfma32(dsp[qt][f / C::NDT], fr, dq[qt][f % C::NDT]);
        }
    };

    if (steps.next_block()) {
        int n0 = steps.n0;                         // step t
        plan(n0, 0);
#pragma unroll
        for (int k = 0; k < C::NL; ++k) fire(k);
        bool have1 = steps.next();                 // step t + 1
        int n1 = steps.n0;
        if (have1) plan(n1, 1);
        else restage(1);
#pragma unroll
        for (int k = 0; k < C::NL; ++k) fire(k);
        bool have2 = have1 && steps.next();        // step t + 2
        int n2 = steps.n0;
        wait_vmcnt<C::NL>();                       // this wave's loads of step t landed
        __syncthreads();
        if (have2) plan(n2, 2);
        else restage(2);
        f32x16_t st[C::QT], dpt[C::QT];
        bf16x8_t dsn[C::QT][2];
        sdp(0, st, dpt);
        ds_step(std::false_type{}, 0, st, dpt, n0, dsn, tok_word(0));
#pragma unroll
        for (int qt = 0; qt < C::QT; ++qt) {
            dsp[qt][0] = dsn[qt][0];
            dsp[qt][1] = dsn[qt][1];
        }
        int t = 0;
        while (have1) {
            ++t;
            n0 = n1;
            const bool have3 = have2 && steps.next();
            const int n3 = steps.n0;
            wait_vmcnt<C::NL>();
            __syncthreads();
            if (have3) plan(n3, (t + 2) % C::NS);
            else restage((t + 2) % C::NS);
            sdp(t % C::NS, st, dpt);
            ds_step(std::true_type{}, (t + C::NS - 1) % C::NS, st, dpt, n0, dsn, tok_word(t % C::NS));
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt) {
                dsp[qt][0] = dsn[qt][0];
                dsp[qt][1] = dsn[qt][1];
            }
            have1 = have2;
            n1 = n2;
            have2 = have3;
            n2 = n3;
        }
        wait_vmcnt<0>();                           // no load may land in LDS after the workgroup ends
        dq_last(t % C::NS);
    }

    uint16_t* gdq = a.dq + b * a.dq_sb + h * a.dq_sh;
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m_base + wrow + 32 * qt + 8 * (i >> 2) + 4 * h2 + (i & 3);
                if (m < a.Sq) gdq[m * a.dq_ss + 32 * dt + l32] = to_bf16(dq[qt][dt][i] * a.scale);
            }
}

// ---------------------------------------------------------------------------
// dK/dV pass
//
// One workgroup per (batch, KV head, 128-key block), eight waves in two roles;
// the SIMD that runs P wave r also runs dS wave r, so each one's arithmetic
// fills the other's MFMA gaps:
//   P waves 0-3, 32 keys each: K rows resident in registers, dV accumulators.
//     Step t: S = Q_t K^T and P_t = exp2(S * scale * log2e - lse2), handed to
//     the partner through LDS; the dV += P_{t-1}^T dO_{t-1} MFMAs of the
//     previous step are issued between the P arithmetic.
//   dS waves 4-7, the same keys: V rows resident, dK accumulators.  Step t
//     finishes query slice t-1: dP = dO V^T, dS = P (dP - delta) with P from
//     the partner, dK += dS^T Q.
// A step is BM query rows of one kept query block of one head of the GQA
// group.  The Q/dO tiles and the rows' lse2/delta go through a 3-stage LDS
// ring filled by direct global->LDS loads issued one step ahead.
// ---------------------------------------------------------------------------
template <int DQK, int DV>
struct DkvCfg {
    static constexpr int BN = 128;                          // keys per workgroup
    static constexpr int BM = 64;                           // query rows per step (one LDS stage)
    static constexpr int NH = 2;                            // 32-row halves a wave computes per step
    static constexpr int NW = 8;
    static constexpr int NT = 64 * NW;
    static constexpr int NR = NW / 2;                       // waves per role (32 keys each)
    static constexpr int NS = 3;                            // LDS ring stages (loads run one step ahead)
    static constexpr int Q_BYTES = BM * DQK * 2;
    static constexpr int O_BYTES = BM * DV * 2;
    static constexpr int ST_BYTES = 2 * BM * 4;             // float lse2[64], -delta[64]
    static constexpr int XBUF_BYTES = NR * NH * 2 * 1024;   // P of all P waves for one step, (wave, half, cc)
    // LDS regions: the NS Q tiles, the NS dO tiles, the NS statistics slots,
    // two P buffers
    static constexpr int Q_OFF = 0;
    static constexpr int O_OFF = Q_OFF + NS * Q_BYTES;
    static constexpr int S_OFF = O_OFF + NS * O_BYTES;
    static constexpr int X_OFF = S_OFF + NS * ST_BYTES;
    // token-exact masks: each P wave's 32 keys' bit words of the step's 64
    // rows (64 lanes x 4 B), per stage
    static constexpr int TK_STAGE = NR * 256;
    static constexpr int T_OFF = X_OFF + 2 * XBUF_BYTES;
    static constexpr int LDS_BYTES = T_OFF + NS * TK_STAGE;
    static constexpr int HQ = 32 * DQK * 2;                 // bytes of 32 Q rows
    static constexpr int HO = 32 * DV * 2;
    static constexpr int NQI = Q_BYTES / 1024;              // 1 KiB loads per Q tile
    static constexpr int NI = (Q_BYTES + O_BYTES) / 1024;   // 1 KiB loads per step
    // Where the registers allow (Dqk <= 128) only the P waves load, so the
    // dS waves never wait on the memory counter at a step barrier; else all
    // eight waves share the tile loads and the dS waves load the statistics.
    static constexpr bool P_LOADS = DQK <= 128;
    static constexpr int NLW = P_LOADS ? NR : NW;           // waves sharing the tile loads
    static constexpr int KMAX = (NI + NLW - 1) / NLW;       // tile loads per loading wave per step
    static constexpr int NDMA_P = P_LOADS ? KMAX + 1 : KMAX;   // loads a P wave issues per step
    static constexpr int NDMA_S = P_LOADS ? 0 : KMAX + 1;      // loads a dS wave issues per step
    static constexpr int NCQ = DQK / 16;
    static constexpr int NCV = DV / 16;
    static constexpr int NDK = DQK / 32;
    static constexpr int NDV = DV / 32;
    static_assert(BM == 64, "one statistics load (64 lanes) covers a step");
    static_assert(Q_BYTES % 1024 == 0 && O_BYTES % 1024 == 0, "tiles split into whole wave loads");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert((NH - 1) * HQ + 48 * DQK * 2 < 65536 && (NH - 1) * HO + 48 * DV * 2 < 65536,
                  "row-group offsets fit the LDS instruction offset field");
    static_assert(NDMA_P + 1 <= NH * NCQ && NDMA_S <= NCV, "loads must fit between the MFMAs");
};

// Step sequence of one workgroup: every BM-row part of every kept query
// block of every head of the GQA group.  Every wave walks it identically.
// Visibility (causal) is decided per block; parts of a visible block that no
// row of sees, or that lie past Sq, are still stepped through: their P is
// masked to zero or their rows' lse2 is +inf.
//
// The kept query blocks of a head are taken 64 list entries at a time, one
// per lane: each lane decides its entry (in the item's [lo, hi) range, a
// valid block index, some row of it sees the key block) and computes its dS
// tile slot, and the valid entries are packed to the low lanes in list
// order (ballot, prefix popcount, ds_permute).  A step then reads its block
// and slot with two lane reads; the per-entry tests run once per 64 entries,
// lane-parallel, instead of serially at every step.
template <int BM, bool DS>
struct DkvSteps {
    static constexpr int PARTS = kBlock / BM;
    const BwdArgs& a;
    int b, hk, kb, n_base, shift, lane;
    int gi = 0, part = 0, count = 0, first = 0;
    int m = 0;                                      // first row of the current step
    int cum = 0;                                    // blocks in the group's earlier heads
    int lo = 0, hi = INT_MAX;                       // range of the group's concatenated block lists
    int scan = 0;                                   // next list entry of the current head to take
    int pos = 0, nval = 0;                          // current / number of packed entries
    int e_qb = 0;                                   // packed entries (one per lane): block, dS slot
    int e_tile = 0;
    const int32_t* list = nullptr;
    // DS (SPLIT_DS): the dS tile slot (dS tile slots in bwd_args.hpp) of the
    // current block, and the current head's slot of its first list entry
    // (block CSR: R * the K->Q position + the head's place among the R query
    // heads of its mask head; the next entry is R slots on) or of (qb = 0,
    // kb) (dense)
    int tile = 0, tile0 = 0;
    // the current head's Q, dO and statistics rows
    const uint16_t* qh = nullptr;
    const uint16_t* oh = nullptr;
    const float* lh = nullptr;
    const float* dh = nullptr;

    __device__ DkvSteps(const BwdArgs& a_, int b_, int hk_, int kb_, int lane_)
        : a(a_), b(b_), hk(hk_), kb(kb_), n_base(kb_ * kBlock), shift(a_.Sk - a_.Sq), lane(lane_) {}

    __device__ int hq() const { return hk * a.G + gi; }
    // element offset of the current step's part of its dS tile (SPLIT_DS):
    // the 128 x 128 bf16 tile of the block's slot, the step's 64 rows its
    // half m % 128 / 64 (only the dS waves of SPLIT_DS use it)
    __device__ int64_t ds_off() const { return int64_t(tile) * (kBlock * kBlock) + (m % kBlock) * kBlock; }

    __device__ void load_head() {
        const int h = hq();
        qh = a.q + b * a.q_sb + h * a.q_sh;
        oh = a.dO + b * a.do_sb + h * a.do_sh;
        const int64_t srow = (int64_t(b) * a.Hq + h) * a.stat_ld;
        lh = a.lse2 + srow;
        dh = a.delta + srow;
        list = nullptr;
        first = 0;
        if (a.mask_kind == 1) {
            const int hm = h * a.Hm / a.Hq;
            const int r = (b * a.Hm + hm) * a.n_kb + kb;
            const int beg = a.k2q_ptr[r];
            count = a.k2q_ptr[r + 1] - beg;
            list = a.k2q_col + beg;
            if constexpr (DS) {
                const int R = a.Hq / a.Hm;
                tile0 = R * beg + (h - hm * R);
            }
        } else {
            if (a.causal) {
                const int first_row = n_base - shift;
                first = first_row <= 0 ? 0 : first_row / kBlock;
            }
            count = (a.Sq + kBlock - 1) / kBlock - first;
            if constexpr (DS) tile0 = (b * a.Hq + h) * a.ds_T + kb;
        }
    }
    // pack the current head's entries scan .. scan + 63 (see above)
    __device__ void refill() {
        const int e = scan + lane;
        bool v = e < count && cum + e < hi;
        int qb = -1;
        if (v) qb = list != nullptr ? list[e] : first + e;
        v = v && qb >= 0 && qb < a.n_qb && qb * kBlock < a.Sq &&                  // a malformed entry: nothing to do
            !(a.causal && min(qb * kBlock + kBlock - 1, a.Sq - 1) + shift < n_base);   // no row sees the key block
        int tl = 0;
        if constexpr (DS) {
            if (v) {
                if (list != nullptr) tl = tile0 + (a.Hq / a.Hm) * e;
                else tl = tile0 + (a.cu_q != nullptr ? qb * a.n_kb
                                                      : int(visible_before(qb, a.Sq, a.Sk, a.n_kb, a.causal != 0)));
            }
        }
        const uint64_t mask = __ballot(v);
        const int dst = v ? __popcll(mask & ((uint64_t(1) << lane) - 1)) : 63;   // unused lanes: slot 63, past nval
        e_qb = __builtin_amdgcn_ds_permute(dst * 4, qb);
        if constexpr (DS) e_tile = __builtin_amdgcn_ds_permute(dst * 4, tl);
        nval = __popcll(mask);
        pos = -1;
        scan += 64;
    }
    // next kept block some row of which sees the key block; false at the end
    // (of the item, or of its [lo, hi) range)
    __device__ bool next_block() {
        for (;;) {
            if (++pos < nval) {
                const int qb = __builtin_amdgcn_readlane(e_qb, pos);
                if constexpr (DS) tile = __builtin_amdgcn_readlane(e_tile, pos);
                part = 0;
                m = qb * kBlock;
                return true;
            }
            while (scan >= count) {                 // the head's list is done
                if (++gi >= a.G) return false;
                cum += count;
                load_head();
                scan = 0;
            }
            if (cum + scan >= hi) return false;
            refill();
        }
    }
    __device__ bool start() {
        load_head();
        while (cum + count <= lo) {                 // heads entirely before the range
            if (++gi >= a.G) return false;
            cum += count;
            load_head();
        }
        scan = lo - cum;
        pos = 0;
        nval = 0;
        return next_block();
    }
    __device__ bool next() {
        if (++part < PARTS) {
            m += BM;
            return true;
        }
        return next_block();
    }
};

// A ring position: which of the NS stages a role's reads point at.  advance()
// moves to the next stage and returns the byte distance in units of one
// stage (+1, or 1 - NS at the wrap).
template <int NS>
struct RingPos {
    int s;
    __device__ int advance() {
        const int n = s == NS - 1 ? 0 : s + 1;
        const int d = n - s;
        s = n;
        return d;
    }
};

template <int DQK, int DV>
struct DkvShared {
    using C = DkvCfg<DQK, DV>;
    const BwdArgs& a;
    uint16_t* lds;
    uint32_t lds_base;
    const lds_char* lp;                             // the LDS window as an LDS pointer
    int w, lane, l32, h2, b, hk, n_base;
    uint32_t toff[C::KMAX];                         // per-lane byte offsets of this wave's tile loads (no clamping)
    uint32_t soff;                                  // per-lane byte offset of the statistics load

    // The loads of one step: wave-uniform source pointers (a head's rows) and
    // LDS destinations (Q tile, dO tile, statistics slot of the stage),
    // per-lane byte offsets (the step's rows included).
    struct Dma {
        const uint16_t* q;
        const uint16_t* o;
        const float* st;
        const uint32_t* tk;                         // token words of the step (P waves, token masks)
        uint32_t lq, lo, ls, lt;
        uint32_t off[C::KMAX];
        uint32_t soff;
    };

    // 1 KiB tile load k of loading wave w: instruction j = w + NLW * k of the
    // step's Q tile (j < NQI) then dO tile; a j past the last re-issues
    // j - NLW, which writes the same bytes again.
    static __device__ int load_index(int w, int k) {
        const int j = w + C::NLW * k;
        return j < C::NI ? j : j - C::NLW;
    }

    __device__ DkvShared(const BwdArgs& a_, uint16_t* lds_, int w_, int lane_, int b_, int hk_, int n_base_)
        : a(a_), lds(lds_), lds_base(lds_address(lds_)), lp(lds_ptr(lds_)), w(w_), lane(lane_), l32(lane_ & 31),
          h2(lane_ >> 5), b(b_), hk(hk_), n_base(n_base_) {
#pragma unroll
        for (int k = 0; k < C::KMAX; ++k) toff[k] = load_off(load_index(w, k), C::BM);
        soff = uint32_t(4 * swap23(lane));         // LDS position L holds row swap23(L) of the step
    }
    // byte offset of this lane's 16 bytes in 1 KiB load j (Q or dO part) of a
    // swizzled tile (tile row t at LDS row swap23(t)); rows past `lim` read row lim
    template <int D>
    __device__ uint32_t tile_off(int jj, int lim, int64_t ss) const {
        const int e = 512 * jj + 8 * lane;
        const int r = e / D;
        const int c = ((e - r * D) >> 3) ^ chunk_swz(r, D);
        return uint32_t(min(swap23(r), lim)) * uint32_t(ss * 2) + uint32_t(16 * c);
    }
    __device__ uint32_t load_off(int j, int lim) const {
        return j < C::NQI ? tile_off<DQK>(j, lim, a.q_ss) : tile_off<DV>(j - C::NQI, lim, a.do_ss);
    }

    // Plan the loads of the steps' current step into stage s.
    template <bool TOK, bool DS>
    __device__ void plan(Dma& d, const DkvSteps<C::BM, DS>& st, int s) const {
        const int m = st.m;
        restage(d, s);
        d.q = st.qh;
        d.o = st.oh;
        if constexpr (TOK) {                        // key-major words of slot (b, mask head, qb, kb), rows m..m+63
            const int h = st.hq();
            d.tk = a.tok + ((int64_t(b) * a.Hm + h * a.Hm / a.Hq) * a.n_qb + m / kBlock) * int64_t(a.n_kb) * 1024 +
                   int64_t(n_base / kBlock) * 1024 + 512 + (m % kBlock) / 32;
        }
        d.st = (w & 1) == 0 ? st.lh : st.dh;
        d.soff = soff + uint32_t(4 * m);
        if (m + C::BM <= a.Sq) {
            const uint32_t mq = uint32_t(m) * uint32_t(a.q_ss * 2), mo = uint32_t(m) * uint32_t(a.do_ss * 2);
#pragma unroll
            for (int k = 0; k < C::KMAX; ++k) d.off[k] = toff[k] + (load_index(w, k) < C::NQI ? mq : mo);
        } else {                                    // ragged tail: rows past Sq re-read row Sq - 1
            const int mb = min(m, a.Sq - 1);
            const uint32_t mq = uint32_t(mb) * uint32_t(a.q_ss * 2), mo = uint32_t(mb) * uint32_t(a.do_ss * 2);
#pragma unroll
            for (int k = 0; k < C::KMAX; ++k) {
                const int j = load_index(w, k);
                d.off[k] = load_off(j, a.Sq - 1 - mb) + (j < C::NQI ? mq : mo);
            }
        }
    }
    // Point a plan at another stage (re-loads its rows there).
    __device__ void restage(Dma& d, int s) const {
        d.lq = lds_base + uint32_t(C::Q_OFF + s * C::Q_BYTES);
        d.lo = lds_base + uint32_t(C::O_OFF + s * C::O_BYTES);
        d.ls = lds_base + uint32_t(C::S_OFF + s * C::ST_BYTES);
        d.lt = lds_base + uint32_t(C::T_OFF + s * C::TK_STAGE);
    }

    // Load k of this wave (k < KMAX: tile part; k == KMAX: the step's 64
    // statistics values, by the P waves or the dS waves -- lse2 by even
    // waves, delta by odd ones).
    // With token masks a P wave's last load (k == KMAX + 1 where the P waves
    // load the statistics, else KMAX) is its keys' token words: lane L takes
    // word L / 32 of key 32 w + L % 32.
    // Tile load K where every loading wave's loads split evenly between the
    // Q and dO tiles: wave w's piece K lands 1 KiB x (w + NLW K) into its
    // tile, the wave part added at run time, the rest an immediate.
    template <int K>
    __device__ void fire_tile(const Dma& d) const {
        constexpr bool is_q = C::NLW * K < C::NQI;
        constexpr int imm = 1024 * (is_q ? C::NLW * K : C::NLW * K - C::NQI);
        dma16_imm<imm>(is_q ? d.q : d.o, d.off[K], (is_q ? d.lq : d.lo) + uint32_t(1024 * w));
    }
    template <int... Ks>
    __device__ void fire_tiles(const Dma& d, int k, std::integer_sequence<int, Ks...>) const {
        ((k == Ks ? fire_tile<Ks>(d) : void()), ...);   // k is a constant at every call site
    }
    __device__ void fire(const Dma& d, int k) const {
        if (k < C::KMAX && C::NQI % C::NLW == 0 && C::NI % C::NLW == 0) {
            fire_tiles(d, k, std::make_integer_sequence<int, C::KMAX>{});
        } else if (k < C::KMAX) {
            const int j = load_index(w, k);
            const bool is_q = j < C::NQI;
            dma16(is_q ? d.q : d.o, d.off[k], is_q ? d.lq + uint32_t(1024 * j) : d.lo + uint32_t(1024 * (j - C::NQI)));
        } else if (k == C::KMAX && (C::P_LOADS || w >= C::NR)) {
            dma4(d.st, d.soff, d.ls + uint32_t((w & 1) * 256));
        } else {
            dma4(d.tk, uint32_t(4 * (4 * (32 * w + l32) + h2)), d.lt + uint32_t(256 * w));
        }
    }
};

// P wave: S, P, dV for 32 keys.  Reads: Q rows of the step's stage (S),
// dO^T of the previous step's stage (dV), lse2 of the step; writes P to the
// step's P buffer.
template <int DQK, int DV, bool TOK>
struct DkvPWave {
    static constexpr bool kLoads = true;            // issues the step's tile and statistics loads
    static constexpr bool kTok = TOK;               // and its keys' token words
    using C = DkvCfg<DQK, DV>;
    static constexpr int NDMA = C::NDMA_P + (TOK ? 1 : 0);
    using Dma = typename DkvShared<DQK, DV>::Dma;
    static constexpr int NF = 2 * C::NDV;           // dO^T fragments (cc, j) of one half
    const DkvShared<DQK, DV>& sh;
    const BwdArgs& a;
    int wr;
    bf16x8_t kB[C::NCQ];                            // K rows of the wave's 32 keys
    f32x16_t dv[C::NDV];
    int qmin;                                       // first query row that sees the lane's key
    u32x4_t npp[C::NH][2];                          // P of the step just computed (half, cc), for its dV update
    // read / write addresses: Q rows (chunk pair c) and lse2 at stage qs, dO^T
    // (column group j, lo / hi) at stage os, P buffer of parity par
    const lds_char* qa_at[C::NCQ];
    const lds_char* ot_at[C::NDV][2];
    const lds_char* l_at;
    const lds_char* x_at;
    const lds_char* t_at;                           // token words of this lane's key at stage qs (TOK)
    RingPos<C::NS> qs{0}, os{C::NS - 1};
    int par = 0;

    __device__ DkvPWave(const DkvShared<DQK, DV>& sh_, int wr_) : sh(sh_), a(sh_.a), wr(wr_) {
        const int key = sh.n_base + 32 * wr + sh.l32;
        const bool in = key < a.Sk;
        const uint16_t* kr = a.k + sh.b * a.k_sb + sh.hk * a.k_sh + int64_t(in ? key : 0) * a.k_ss + 8 * sh.h2;
#pragma unroll
        for (int c = 0; c < C::NCQ; ++c) kB[c] = in ? gload_operand(kr + 16 * c) : bf16x8_t{};
        qmin = in ? (a.causal ? key - (a.Sk - a.Sq) : -(1 << 30)) : INT_MAX;   // rows < 2^30: no overflow below
#pragma unroll
        for (int j = 0; j < C::NDV; ++j) dv[j] = f32x16_t{};
        const lds_char* q0 = sh.lp + C::Q_OFF;
        const lds_char* o0 = sh.lp + C::O_OFF + (C::NS - 1) * C::O_BYTES;
#pragma unroll
        for (int c = 0; c < C::NCQ; ++c) qa_at[c] = q0 + row_read_off<DQK>(sh.lane, c);
#pragma unroll
        for (int j = 0; j < C::NDV; ++j)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) ot_at[j][hi] = o0 + tr_read_off<DV>(sh.lane, j, hi);
        l_at = sh.lp + C::S_OFF + 16 * sh.h2;
        x_at = sh.lp + C::X_OFF + wr * C::NH * 2 * 1024 + 16 * sh.lane;
        t_at = sh.lp + C::T_OFF + wr * 256 + 4 * sh.l32;
    }

    // next step: every read moves one stage on, the P buffer flips
    __device__ void advance() {
        const int kq = qs.advance(), ko = os.advance();
        t_at += kq * C::TK_STAGE;
#pragma unroll
        for (int c = 0; c < C::NCQ; ++c) qa_at[c] += kq * C::Q_BYTES;
#pragma unroll
        for (int j = 0; j < C::NDV; ++j) {
            ot_at[j][0] += ko * C::O_BYTES;
            ot_at[j][1] += ko * C::O_BYTES;
        }
        l_at += kq * C::ST_BYTES;
        x_at += par ? -C::XBUF_BYTES : C::XBUF_BYTES;
        par ^= 1;
    }

    __device__ bf16x8_t q_row(int hh, int c) const { return as_bf16x8(lds_ld128(qa_at[c] + hh * C::HQ)); }
    __device__ bf16x8_t dot_frag(int hh, int f) const {   // f = (cc, j)
        const int off = (32 * hh + 16 * (f / C::NDV)) * DV * 2;
        const u32x2_t lo = lds_ld_tr16(ot_at[f % C::NDV][0] + off);
        const u32x2_t hi = lds_ld_tr16(ot_at[f % C::NDV][1] + off);
        const u32x4_t v = {lo[0], lo[1], hi[0], hi[1]};
        return as_bf16x8(v);
    }

    // One step, two 32-row halves: S and P (to the P buffer, read by the
    // partner); with PREV, the dV MFMAs of the same half of the previous step
    // (its P kept in npp) are issued between the P arithmetic.  Masked steps
    // fix the packed P up afterwards.
    template <bool PREV>
    __device__ void body(int m, bool mask, const Dma& d) {
        u32x4_t pn[C::NH][2];
        // Q row operands of the S MFMAs, a ring PF chunks deep; the next
        // half's first PF chunks are read during this half's dV MFMAs
        constexpr int PF = 4;
        bf16x8_t qa[PF];
#pragma unroll
        for (int c = 0; c < PF && c < C::NCQ; ++c) qa[c] = q_row(0, c);
#pragma unroll
        for (int hh = 0; hh < C::NH; ++hh) {
            constexpr int PFD = 2;                  // dO^T fragments read this many ahead
            bf16x8_t fr[PFD + 1];
            if (PREV) {
#pragma unroll
                for (int f = 0; f < PFD; ++f) fr[f] = dot_frag(hh, f);
            }
            f32x16_t st = f32x16_t{};
            {
                // S MFMAs; this wave's loads for the next step go out between them
#pragma unroll
                for (int c = 0; c < C::NCQ; ++c) {
                    st = mfma32(qa[c % PF], kB[c], st);
                    if (c + PF < C::NCQ) qa[c % PF] = q_row(hh, c + PF);
                    if (hh * C::NCQ + c < NDMA) sh.fire(d, hh * C::NCQ + c);
                }
            }
            f32x4_t l4[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) l4[g] = lds_ldf4(l_at + 4 * (32 * hh + 8 * g));

            // dV MFMAs f = (cc, j) of the previous step's half; P pairs q = (cc, jj) between them
            constexpr int NQ = 8;
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                if (f == 2 && hh + 1 < C::NH) {
#pragma unroll
                    for (int c = 0; c < PF && c < C::NCQ; ++c) qa[c] = q_row(hh + 1, c);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (PREV) {
                    if (f + PFD < NF) fr[(f + PFD) % (PFD + 1)] = dot_frag(hh, f + PFD);
                    dv[f % C::NDV] = mfma32(as_bf16x8(npp[hh][f / C::NDV]), fr[f % (PFD + 1)], dv[f % C::NDV]);
                }
#pragma unroll
                for (int q = f * NQ / NF; q < (f + 1) * NQ / NF; ++q) {
                    const int cc = q >> 2, jj = q & 3;
                    float p2[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int i = 8 * cc + 2 * jj + e;
                        const f32x4_t lv = l4[i >> 2];
                        const float l = (i & 3) == 0 ? lv.x : (i & 3) == 1 ? lv.y : (i & 3) == 2 ? lv.z : lv.w;
                        p2[e] = fast_exp2(fmaf(st[i], a.scale_log2, -l));
                    }
                    pn[hh][cc][jj] = pack_bf16x2(p2[0], p2[1]);
                    if (jj == 3) lds_st128(x_at + (hh * 2 + cc) * 1024, pn[hh][cc]);
                }
            }
        }
        if (mask) {
            // pairs whose row is below the lane key's first visible row (causal),
            // whose key is past Sk, or (token masks) whose row did not select the
            // key: clear the bf16 halves and rewrite
            uint32_t tw[C::NH] = {~0u, ~0u};
            if constexpr (TOK) {
                tw[0] = *(const __attribute__((address_space(3))) uint32_t*)(t_at) >> (8 * sh.h2);
                tw[1] = *(const __attribute__((address_space(3))) uint32_t*)(t_at + 128) >> (8 * sh.h2);
            }
#pragma unroll
            for (int hh = 0; hh < C::NH; ++hh) {
                const int tau = qmin - m - 32 * hh - 8 * sh.h2;   // first visible row offset of this lane
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int o = 16 * cc + 2 * jj;
                        uint32_t keep = (o >= tau ? 0x0000ffffu : 0u) | (o + 1 >= tau ? 0xffff0000u : 0u);
                        if constexpr (TOK)
                            keep &= (((tw[hh] >> o) & 1u) ? 0x0000ffffu : 0u) | (((tw[hh] >> (o + 1)) & 1u) ? 0xffff0000u : 0u);
                        pn[hh][cc][jj] &= keep;
                    }
                    lds_st128(x_at + (hh * 2 + cc) * 1024, pn[hh][cc]);
                }
            }
        }
#pragma unroll
        for (int hh = 0; hh < C::NH; ++hh) {
            npp[hh][0] = pn[hh][0];
            npp[hh][1] = pn[hh][1];
        }
    }

    __device__ void first(int m, bool mask, const Dma& d, int64_t) { body<false>(m, mask, d); }
    __device__ void step(int m, bool mask, const Dma& d, int64_t) { body<true>(m, mask, d); }
    __device__ void fire_all(const Dma& d) const {
#pragma unroll
        for (int k = 0; k < NDMA; ++k) sh.fire(d, k);
    }
    // dV update of the last step (its dO^T reads at the stage advance() moved to)
    __device__ void drain() {
#pragma unroll
        for (int hh = 0; hh < C::NH; ++hh)
#pragma unroll
            for (int f = 0; f < NF; ++f)
                dv[f % C::NDV] = mfma32(as_bf16x8(npp[hh][f / C::NDV]), dot_frag(hh, f), dv[f % C::NDV]);
    }
    __device__ void store(float* partial) const {
        if (partial != nullptr) {                   // fp32 partial dV: slot columns Dqk ..
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int n = 32 * wr + 8 * (i >> 2) + 4 * sh.h2 + (i & 3);
#pragma unroll
                for (int j = 0; j < C::NDV; ++j) partial[n * (DQK + DV) + DQK + 32 * j + sh.l32] = dv[j][i];
            }
            return;
        }
        uint16_t* g = a.dv + sh.b * a.dv_sb + sh.hk * a.dv_sh;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int n = sh.n_base + 32 * wr + 8 * (i >> 2) + 4 * sh.h2 + (i & 3);
            if (n < a.Sk) {
#pragma unroll
                for (int j = 0; j < C::NDV; ++j) g[n * a.dv_ss + 32 * j + sh.l32] = to_bf16(dv[j][i]);
            }
        }
    }
};

// dS wave: dP, dS, dK for 32 keys, one step behind the P waves.  Reads: dO
// rows (dP), Q^T (dK), delta and the partner's P, all of the previous step.
template <int DQK, int DV, bool DS>
struct DkvSWave {
    static constexpr bool kLoads = DkvCfg<DQK, DV>::NDMA_S > 0;
    static constexpr bool kTok = false;
    using C = DkvCfg<DQK, DV>;
    using Dma = typename DkvShared<DQK, DV>::Dma;
    const DkvShared<DQK, DV>& sh;
    const BwdArgs& a;
    int wr;
    bf16x8_t vB[C::NCV];
    f32x16_t dk[C::NDK];
    // read addresses: dO rows (chunk pair c), Q^T (column group j, lo / hi)
    // and delta at stage ss, P buffer of parity par
    const lds_char* oa_at[C::NCV];
    const lds_char* qt_at[C::NDK][2];
    const lds_char* d_at;
    const lds_char* x_at;
    RingPos<C::NS> ss{C::NS - 1};
    int par = 1;
    int64_t ds_prev = 0;                            // dS tile part of the step being finished (DS)

    // DS: store the packed dS of half hh (this lane: key 32 wr + l32, query
    // rows 32 hh + 16 cc + 8 h2 + 0..7 of the step) as two 1 KiB chunks, each
    // written whole by one instruction: chunk (wr, hh, cc) of the step's
    // half tile, lane L at 16 L.  Non-temporal: nothing here reads it again.
    __device__ void store_ds(int hh, const u32x4_t (&sa)[2]) const {
        if constexpr (DS) {
            uint16_t* dst = a.ds + ds_prev + ((wr * 2 + hh) * 2) * 512 + 8 * sh.lane;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
                __builtin_nontemporal_store(sa[cc], reinterpret_cast<u32x4_t*>(dst + 512 * cc));
        }
    }

    __device__ DkvSWave(const DkvShared<DQK, DV>& sh_, int wr_) : sh(sh_), a(sh_.a), wr(wr_) {
        const int key = sh.n_base + 32 * wr + sh.l32;
        const bool in = key < a.Sk;
        const uint16_t* vr = a.v + sh.b * a.v_sb + sh.hk * a.v_sh + int64_t(in ? key : 0) * a.v_ss + 8 * sh.h2;
#pragma unroll
        for (int c = 0; c < C::NCV; ++c) vB[c] = in ? gload_operand(vr + 16 * c) : bf16x8_t{};
#pragma unroll
        for (int j = 0; j < C::NDK; ++j) dk[j] = f32x16_t{};
        const lds_char* o0 = sh.lp + C::O_OFF + (C::NS - 1) * C::O_BYTES;
        const lds_char* q0 = sh.lp + C::Q_OFF + (C::NS - 1) * C::Q_BYTES;
#pragma unroll
        for (int c = 0; c < C::NCV; ++c) oa_at[c] = o0 + row_read_off<DV>(sh.lane, c);
#pragma unroll
        for (int j = 0; j < C::NDK; ++j)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) qt_at[j][hi] = q0 + tr_read_off<DQK>(sh.lane, j, hi);
        d_at = sh.lp + C::S_OFF + (C::NS - 1) * C::ST_BYTES + 4 * C::BM + 16 * sh.h2;   // delta slot follows lse2
        x_at = sh.lp + C::X_OFF + C::XBUF_BYTES + wr * C::NH * 2 * 1024 + 16 * sh.lane;
    }

    __device__ void advance() {
        const int k = ss.advance();
#pragma unroll
        for (int c = 0; c < C::NCV; ++c) oa_at[c] += k * C::O_BYTES;
#pragma unroll
        for (int j = 0; j < C::NDK; ++j) {
            qt_at[j][0] += k * C::Q_BYTES;
            qt_at[j][1] += k * C::Q_BYTES;
        }
        d_at += k * C::ST_BYTES;
        x_at += par ? -C::XBUF_BYTES : C::XBUF_BYTES;
        par ^= 1;
    }

    __device__ bf16x8_t o_row(int hh, int c) const { return as_bf16x8(lds_ld128(oa_at[c] + hh * C::HO)); }
    __device__ bf16x8_t qt_frag(int hh, int f) const {   // f = (cc, j)
        const int off = (32 * hh + 16 * (f / C::NDK)) * DQK * 2;
        const u32x2_t lo = lds_ld_tr16(qt_at[f % C::NDK][0] + off);
        const u32x2_t hi = lds_ld_tr16(qt_at[f % C::NDK][1] + off);
        const u32x4_t v = {lo[0], lo[1], hi[0], hi[1]};
        return as_bf16x8(v);
    }

    // Initial dP accumulators of a half: the rows' -delta (the statistics
    // slot holds the negated value, four rows per 16-byte read in accumulator
    // order), so the MFMAs leave dP - delta and dS needs one multiply.
    static __device__ f32x16_t neg_delta(const f32x4_t (&d4)[4]) {
        f32x16_t r;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const f32x4_t v = d4[i >> 2];
            r[i] = (i & 3) == 0 ? v.x : (i & 3) == 1 ? v.y : (i & 3) == 2 ? v.z : v.w;
        }
        return r;
    }
    // dS pair (cc, jj): packed bf16 of P * (dP - delta), dpt holding dP - delta
    __device__ uint32_t ds_pair(const f32x16_t& dpt, uint32_t pw, int cc, int jj) const {
        float r[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int i = 8 * cc + 2 * jj + e;
            const float p = e == 0 ? bf16_lo(pw) : bf16_hi(pw);
            r[e] = p * dpt[i];
        }
        return pack_bf16x2(r[0], r[1]);
    }

    // Finish the previous step's query slice as a two-half pipeline that
    // keeps the dS arithmetic under MFMAs: dP(0); dP(1) with dS(0) between
    // its MFMAs; dK(0) with dS(1) between its MFMAs; dK(1).  With FIRE this
    // wave's loads for the next step (if it has any) go out between the dP(0)
    // MFMAs.
    template <bool FIRE>
    __device__ void finish_pipe(const Dma& d) {
#pragma unroll
        for (int j = 0; j < C::NDK; ++j) asm volatile("" : "+v"(dk[j]));
        constexpr int PFO = 4;                      // dO rows read this many ahead
        constexpr int NQF = 2 * C::NDK;             // Q^T fragments (cc, j) of a half
        constexpr int PFQ = 3;                      // Q^T fragments read this many ahead
        static_assert(C::NH == 2, "two 32-row halves per step");
        f32x16_t dp[C::NH];
        f32x4_t d4[C::NH][4];
        u32x4_t pw[C::NH][2];
        u32x4_t sa[C::NH][2];
        auto load_stats = [&](int hh) {
#pragma unroll
            for (int g = 0; g < 4; ++g) d4[hh][g] = lds_ldf4(d_at + 4 * (32 * hh + 8 * g));
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) pw[hh][cc] = lds_ld128(x_at + (hh * 2 + cc) * 1024);
        };
        auto ds_q = [&](int hh, int q) {
            sa[hh][q >> 2][q & 3] = ds_pair(dp[hh], pw[hh][q >> 2][q & 3], q >> 2, q & 3);
        };
        bf16x8_t oa[PFO];
        // dP(0)
#pragma unroll
        for (int c = 0; c < PFO && c < C::NCV; ++c) oa[c] = o_row(0, c);
        load_stats(0);
        dp[0] = neg_delta(d4[0]);
#pragma unroll
        for (int c = 0; c < C::NCV; ++c) {
            dp[0] = mfma32(oa[c % PFO], vB[c], dp[0]);
            if (c + PFO < C::NCV) oa[c % PFO] = o_row(0, c + PFO);
            if (FIRE && c < C::NDMA_S) sh.fire(d, c);
        }
        // dP(1) with dS(0) between its MFMAs
#pragma unroll
        for (int c = 0; c < PFO && c < C::NCV; ++c) oa[c] = o_row(1, c);
        load_stats(1);
        dp[1] = neg_delta(d4[1]);
#pragma unroll
        for (int c = 0; c < C::NCV; ++c) {
            dp[1] = mfma32(oa[c % PFO], vB[c], dp[1]);
            if (c + PFO < C::NCV) oa[c % PFO] = o_row(1, c + PFO);
#pragma unroll
            for (int q = c * 8 / C::NCV; q < (c + 1) * 8 / C::NCV; ++q) ds_q(0, q);
            __builtin_amdgcn_sched_barrier(0);     // one MFMA and its share of the arithmetic together
        }
        store_ds(0, sa[0]);
        // dK(0) with dS(1) between its MFMAs
        bf16x8_t qf[PFQ + 1];
#pragma unroll
        for (int f = 0; f < PFQ; ++f) qf[f] = qt_frag(0, f);
#pragma unroll
        for (int f = 0; f < NQF; ++f) {
            if (f + PFQ < NQF) qf[(f + PFQ) % (PFQ + 1)] = qt_frag(0, f + PFQ);
            else qf[(f + PFQ) % (PFQ + 1)] = qt_frag(1, f + PFQ - NQF);
            dk[f % C::NDK] = mfma32(as_bf16x8(sa[0][f / C::NDK]), qf[f % (PFQ + 1)], dk[f % C::NDK]);
#pragma unroll
            for (int q = f * 8 / NQF; q < (f + 1) * 8 / NQF; ++q) ds_q(1, q);
            __builtin_amdgcn_sched_barrier(0);     // one MFMA and its share of the arithmetic together
        }
        store_ds(1, sa[1]);
        // dK(1)
#pragma unroll
        for (int f = 0; f < NQF; ++f) {
            const int g = NQF + f;                  // fragment index across both halves
            if (f + PFQ < NQF) qf[(g + PFQ) % (PFQ + 1)] = qt_frag(1, f + PFQ);
            dk[f % C::NDK] = mfma32(as_bf16x8(sa[1][f / C::NDK]), qf[g % (PFQ + 1)], dk[f % C::NDK]);
        }
#pragma unroll
        for (int j = 0; j < C::NDK; ++j) asm volatile("" : "+v"(dk[j]));   // the accumulators are not moved
    }

    // The same, half by half (dP, dS, dK per 32-row half): fewer live
    // registers, for Dqk = 192.
    template <bool FIRE>
    __device__ void finish_halves(const Dma& d) {
#pragma unroll
        for (int j = 0; j < C::NDK; ++j) asm volatile("" : "+v"(dk[j]));
#pragma unroll
        for (int hh = 0; hh < C::NH; ++hh) {
            constexpr int PFO = 4;                  // dO rows read this many ahead
            bf16x8_t oa[PFO];
#pragma unroll
            for (int c = 0; c < PFO && c < C::NCV; ++c) oa[c] = o_row(hh, c);
            f32x4_t d4[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) d4[g] = lds_ldf4(d_at + 4 * (32 * hh + 8 * g));
            u32x4_t pw[2];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) pw[cc] = lds_ld128(x_at + (hh * 2 + cc) * 1024);
            constexpr int NQF = 2 * C::NDK;        // Q^T fragments (cc, j)
            bf16x8_t qf[NQF];
            f32x16_t dp = neg_delta(d4);
#pragma unroll
            for (int c = 0; c < C::NCV; ++c) {
                dp = mfma32(oa[c % PFO], vB[c], dp);
                if (c + PFO < C::NCV) oa[c % PFO] = o_row(hh, c + PFO);
                if (FIRE && hh == 0 && c < C::NDMA_S) sh.fire(d, c);
#pragma unroll
                for (int f = c * NQF / C::NCV; f < (c + 1) * NQF / C::NCV; ++f) qf[f] = qt_frag(hh, f);
            }
            u32x4_t sa[2];
#pragma unroll
            for (int q = 0; q < 8; ++q) sa[q >> 2][q & 3] = ds_pair(dp, pw[q >> 2][q & 3], q >> 2, q & 3);
            store_ds(hh, sa);
#pragma unroll
            for (int f = 0; f < NQF; ++f) dk[f % C::NDK] = mfma32(as_bf16x8(sa[f / C::NDK]), qf[f], dk[f % C::NDK]);
        }
#pragma unroll
        for (int j = 0; j < C::NDK; ++j) asm volatile("" : "+v"(dk[j]));   // the accumulators are not moved
    }

    // Finish the previous step's query slice; the two-half pipeline where its
    // registers fit (Dqk <= 128).
    template <bool FIRE>
    __device__ void finish(const Dma& d) {
        if constexpr (DQK <= 128) finish_pipe<FIRE>(d);
        else finish_halves<FIRE>(d);
    }

    __device__ void first(int m, bool mask, const Dma& d, int64_t dso) {
        (void)m;
        (void)mask;
        // the V rows land before the step loop: a wave that issues no loads in
        // the loop (but may store dS) then never waits on the memory counter
        // inside it (the compiler would otherwise guard the first use of vB in
        // the loop body, and that wait would also cover the dS stores)
        wait_vmcnt<0>();
        ds_prev = dso;
        fire_all(d);
    }
    __device__ void step(int m, bool mask, const Dma& d, int64_t dso) {
        (void)m;
        (void)mask;
        finish<true>(d);
        ds_prev = dso;
    }
    __device__ void drain() {
        Dma d{};
        finish<false>(d);
    }
    __device__ void fire_all(const Dma& d) const {
#pragma unroll
        for (int k = 0; k < C::NDMA_S; ++k) sh.fire(d, k);
    }

    __device__ void store(float* partial) const {
        if (partial != nullptr) {                   // fp32 partial dK (unscaled): slot columns 0 .. Dqk
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int n = 32 * wr + 8 * (i >> 2) + 4 * sh.h2 + (i & 3);
#pragma unroll
                for (int j = 0; j < C::NDK; ++j) partial[n * (DQK + DV) + 32 * j + sh.l32] = dk[j][i];
            }
            return;
        }
        uint16_t* g = a.dk + sh.b * a.dk_sb + sh.hk * a.dk_sh;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int n = sh.n_base + 32 * wr + 8 * (i >> 2) + 4 * sh.h2 + (i & 3);
            if (n < a.Sk) {
#pragma unroll
                for (int j = 0; j < C::NDK; ++j) g[n * a.dk_ss + 32 * j + sh.l32] = to_bf16(dk[j][i] * a.scale);
            }
        }
    }
};

// The barrier between steps: a loading wave first waits for its own loads of
// the step (direct-to-LDS, not tracked by the compiler); a wave that issues
// no loads waits only for its LDS accesses, so global stores it has in
// flight do not hold it up.
template <bool LOADS>
__device__ __forceinline__ void step_barrier() {
    if constexpr (LOADS) {
        wait_vmcnt<0>();
        __syncthreads();
    } else {
        __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0); vmcnt and expcnt unconstrained
        __builtin_amdgcn_s_barrier();
    }
}

// Steps, barriers and loads, shared by both roles.  Step t's tiles sit in
// ring stage t % NS; the P waves read stage t, the dS waves stage t - 1; P
// goes to buffer t % 2.  The loads of step t + 1 go out from inside the P
// waves' step t MFMA stream (their stage was last read in step t - 1,
// before the barrier that opens step t); past the last step they re-read the
// last planned step's rows into the free stage, which keeps the step bodies
// free of branches.  The loop body is one straight-line block per role (masking is a
// fix-up on the packed P, outside the MFMA block) so the accumulators stay
// put in registers.
template <int DQK, int DV, bool DS, class Role>
__device__ __forceinline__ void dkdv_run(const DkvShared<DQK, DV>& sh, DkvSteps<DkvCfg<DQK, DV>::BM, DS>& steps,
                                         Role& role) {
    using C = DkvCfg<DQK, DV>;
    const BwdArgs& a = sh.a;
    const bool ragged_keys = sh.n_base + C::BN > a.Sk;
    const int shift = a.Sk - a.Sq;
    // some pair of step m is masked (rows past Sq need no mask: their lse2 is +inf)
    auto need_mask = [&](int m) {
        return Role::kTok || ragged_keys || (a.causal && sh.n_base + C::BN - 1 > m + shift);
    };
    if (!steps.start()) return;
    typename DkvShared<DQK, DV>::Dma d;
    int m = steps.m;                                // step t
    int64_t dso = steps.ds_off();
    sh.template plan<Role::kTok>(d, steps, 0);
    role.fire_all(d);
    bool have1 = steps.next();                      // step t + 1
    int m1 = steps.m;
    int64_t dso1 = steps.ds_off();
    step_barrier<Role::kLoads>();
    if (have1) sh.template plan<Role::kTok>(d, steps, 1);
    else sh.restage(d, 1);
    role.first(m, need_mask(m), d, dso);
    int t = 0;
    while (have1) {
        ++t;
        m = m1;
        dso = dso1;
        const bool have2 = steps.next();
        const int m2 = steps.m;
        const int64_t dso2 = steps.ds_off();
        step_barrier<Role::kLoads>();               // the loads of step t landed
        if (have2) sh.template plan<Role::kTok>(d, steps, (t + 1) % C::NS);
        else sh.restage(d, (t + 1) % C::NS);
        role.advance();
        role.step(m, need_mask(m), d, dso);
        have1 = have2;
        m1 = m2;
        dso1 = dso2;
    }
    step_barrier<Role::kLoads>();                   // no load may land in LDS after the workgroup ends
    role.advance();
    role.drain();
}

template <int DQK, int DV, bool DS, bool VL, bool TOK>
__global__ __launch_bounds__(512, 1) void k_bwd_dkdv(BwdArgs a) {
    using C = DkvCfg<DQK, DV>;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps role and load addresses scalar
    // items (b, KV head, key block) in the per-XCD work order, or in part mode
    // the units (item, part) longest first
    int item, lo = 0, hi = INT_MAX;
    float* partial = nullptr;
    if (a.kv_parts_T > 0) {
        if (int(blockIdx.x) >= a.units[a.kv_units_bound]) return;
        const int unit = a.units[blockIdx.x];
        item = unit >> 6;
        const int part = unit & (kMaxParts - 1);
        const int work = a.item_info[3 * item], parts = a.item_info[3 * item + 1];
        const int len = (work + parts - 1) / parts;
        lo = part * len;
        hi = min(work, lo + len);
        if (parts > 1) partial = a.partial + int64_t(a.item_info[3 * item + 2] + part) * kBlock * (DQK + DV);
    } else {
        const int slot = xcd_item(blockIdx.x, a.n_kb * a.B * a.Hk);
        if (slot < 0) return;
        item = a.order[slot];
    }
    const int bh = item / a.n_kb;
    const int kb = item - bh * a.n_kb;
    const int b = bh / a.Hk;
    const int hk = bh - b * a.Hk;
    if constexpr (VL) {                            // packed sequences: narrow to sequence b
        seq_view(a, b);
        if (kb * C::BN >= a.Sk) return;            // a key block past the end of the sequence
    }
    const DkvShared<DQK, DV> sh(a, lds, w, lane, b, hk, kb * C::BN);
    DkvSteps<C::BM, DS> steps(a, b, hk, kb, lane);
    steps.lo = lo;
    steps.hi = hi;
    // a block CSR whose true block count needs more dS tiles than the
    // workspace holds (flagged by the set-up launch): nothing is computed or
    // stored rather than anything written past the workspace (read once the
    // K / V rows are on their way)
    const bool overflow = DS && a.ds_flag != nullptr && *a.ds_flag != 0;
    if (w < C::NR) {
        DkvPWave<DQK, DV, TOK> role(sh, w);
        if (overflow) {
            wait_vmcnt<0>();
            return;
        }
        dkdv_run<DQK, DV, DS>(sh, steps, role);
        role.store(partial);
    } else {
        DkvSWave<DQK, DV, DS> role(sh, w - C::NR);
        if (overflow) {
            wait_vmcnt<0>();
            return;
        }
        dkdv_run<DQK, DV, DS>(sh, steps, role);
        role.store(partial);
    }
}

template <int DQK, int DV, int WR, bool VL, bool TOK>
hipError_t launch_dq_t(const BwdArgs& a, hipStream_t s) {
    using C = DqCfg<DQK, DV, WR, TOK>;
    const int64_t items = int64_t(a.n_qb) * a.B * a.Hq;
    if (items == 0) return hipSuccess;
    const int64_t grid = int64_t(kXcds) * xcd_items_per(int(items));
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k_bwd_dq<DQK, DV, WR, VL, TOK>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       C::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((k_bwd_dq<DQK, DV, WR, VL, TOK>), dim3(unsigned(grid)), dim3(C::NT), C::LDS_BYTES, s, a);
    return hipGetLastError();
}

// Part mode: dK = scale * sum of the parts' partial dK, dV = sum of the
// partial dV, in part order, for the items cut into more than one part.
// Workgroup (item, 8-key group): thread t covers columns 4t .. 4t+3 of the
// slot rows (dK columns, then dV).
template <int DQK, int DV>
__global__ __launch_bounds__(256) void k_dkdv_reduce(BwdArgs a) {
    constexpr int W = DQK + DV;
    const int item = blockIdx.x / (kBlock / 8);
    if (a.ds_flag != nullptr && *a.ds_flag != 0) return;   // SPLIT_DS overflow: the parts computed nothing
    const int parts = a.item_info[3 * item + 1];
    if (parts <= 1) return;
    const int slot = a.item_info[3 * item + 2];
    const int bh = item / a.n_kb;
    const int kb = item - bh * a.n_kb;
    const int b = bh / a.Hk;
    const int hk = bh - b * a.Hk;
    if (a.cu_q != nullptr) seq_view(a, b);
    const int key0 = (blockIdx.x % (kBlock / 8)) * 8;
    for (int u = threadIdx.x; u < 8 * W / 4; u += 256) {
        const int r = key0 + (4 * u) / W;
        const int c = (4 * u) % W;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (int p = 0; p < parts; ++p)
            acc += *reinterpret_cast<const f32x4_t*>(a.partial + (int64_t(slot + p) * kBlock + r) * W + c);
        const int n = kb * kBlock + r;
        if (n >= a.Sk) continue;
        uint16_t* dst = c < DQK ? a.dk + b * a.dk_sb + hk * a.dk_sh + int64_t(n) * a.dk_ss + c
                                : a.dv + b * a.dv_sb + hk * a.dv_sh + int64_t(n) * a.dv_ss + (c - DQK);
        const float mul = c < DQK ? a.scale : 1.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = to_bf16(acc[e] * mul);
    }
}

template <int DQK, int DV, bool DS, bool VL, bool TOK>
hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t s) {
    using C = DkvCfg<DQK, DV>;
    const int64_t items = int64_t(a.n_kb) * a.B * a.Hk;
    if (items == 0) return hipSuccess;
    const int64_t grid = int64_t(kXcds) * xcd_items_per(int(items));
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k_bwd_dkdv<DQK, DV, DS, VL, TOK>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       C::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    if (a.kv_parts_T > 0) {                        // part mode: one workgroup per unit, then the reduction
        hipLaunchKernelGGL((k_bwd_dkdv<DQK, DV, DS, VL, TOK>), dim3(unsigned(a.kv_units_bound)), dim3(C::NT), C::LDS_BYTES, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((k_dkdv_reduce<DQK, DV>), dim3(unsigned(items * (kBlock / 8))), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_bwd_dkdv<DQK, DV, DS, VL, TOK>), dim3(unsigned(grid)), dim3(C::NT), C::LDS_BYTES, s, a);
    return hipGetLastError();
}

template <int DQK, int DV, bool TOK>
hipError_t launch_dkdv_v(const BwdArgs& a, hipStream_t s) {
    const bool ds = a.ds != nullptr;               // SPLIT_DS: also store dS
    if (a.cu_q != nullptr)                         // packed sequences
        return ds ? launch_dkdv_t<DQK, DV, true, true, TOK>(a, s) : launch_dkdv_t<DQK, DV, false, true, TOK>(a, s);
    return ds ? launch_dkdv_t<DQK, DV, true, false, TOK>(a, s) : launch_dkdv_t<DQK, DV, false, false, TOK>(a, s);
}

template <int DQK, int DV>
hipError_t launch_dkdv_d(const BwdArgs& a, hipStream_t s) {
    return a.tok != nullptr ? launch_dkdv_v<DQK, DV, true>(a, s) : launch_dkdv_v<DQK, DV, false>(a, s);
}

template <int DQK, int DV, int WR>
hipError_t launch_dq_d(const BwdArgs& a, hipStream_t s) {
    if (a.tok != nullptr)
        return a.cu_q != nullptr ? launch_dq_t<DQK, DV, WR, true, true>(a, s) : launch_dq_t<DQK, DV, WR, false, true>(a, s);
    return a.cu_q != nullptr ? launch_dq_t<DQK, DV, WR, true, false>(a, s) : launch_dq_t<DQK, DV, WR, false, false>(a, s);
}

}  // namespace

hipError_t launch_split_setup(const BwdArgs& a, bool delta, hipStream_t s) {
    const bool sched = int64_t(a.B) * (int64_t(a.Hk) * a.n_kb + int64_t(a.Hq) * a.n_qb) != 0;
    const int32_t n_sched = sched ? 2 * kXcds : 0;
    // the map (and its overflow flag) whenever SPLIT_DS has a block CSR, even an empty one
    const int64_t map_rows = int64_t(a.B) * a.Hm * a.n_qb;
    constexpr int kMapRows = kSchedThreads / 64;
    const int32_t n_map = a.ds_flag != nullptr ? int32_t(max(int64_t(1), (map_rows + kMapRows - 1) / kMapRows)) : 0;
    const int64_t rows = delta ? int64_t(a.B) * a.Hq * a.stat_ld : 0;
    int64_t grid = n_sched + n_map;
    if (rows == 0 || a.Dv == 0) {
        if (grid == 0) return hipSuccess;
        hipLaunchKernelGGL(k_split_setup<0>, dim3(unsigned(grid)), dim3(kSchedThreads), 0, s, a, n_sched, n_map);
    } else if (a.Dv == 64) {
        grid += (rows + delta_rows_per_block<64, kSchedThreads>() - 1) / delta_rows_per_block<64, kSchedThreads>();
        hipLaunchKernelGGL(k_split_setup<64>, dim3(unsigned(grid)), dim3(kSchedThreads), 0, s, a, n_sched, n_map);
    } else if (a.Dv == 128) {
        grid += (rows + delta_rows_per_block<128, kSchedThreads>() - 1) / delta_rows_per_block<128, kSchedThreads>();
        hipLaunchKernelGGL(k_split_setup<128>, dim3(unsigned(grid)), dim3(kSchedThreads), 0, s, a, n_sched, n_map);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_split_dkdv(const BwdArgs& a, hipStream_t s) {
    if (a.Dqk == 64 && a.Dv == 64) return launch_dkdv_d<64, 64>(a, s);
    if (a.Dqk == 128 && a.Dv == 128) return launch_dkdv_d<128, 128>(a, s);
    if (a.Dqk == 192 && a.Dv == 128) return launch_dkdv_d<192, 128>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_split_dq(const BwdArgs& a, hipStream_t s) {
    if (a.Dqk == 64 && a.Dv == 64) return launch_dq_d<64, 64, 32>(a, s);
    if (a.Dqk == 128 && a.Dv == 128) return launch_dq_d<128, 128, 32>(a, s);
    if (a.Dqk == 192 && a.Dv == 128) return launch_dq_d<192, 128, 32>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace isattn
