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
// query rows.  Per 64-key step: S^T = K Q^T and dP^T = V dO^T (A = K/V from
// LDS, B = Q/dO held in registers), P and dS in registers, dQ += dS K with dS
// taken straight from the accumulators and K read back with transposing LDS
// loads.  K/V rows are staged at LDS row swap23(r), which makes each lane's
// accumulator registers cover 8 consecutive keys.
//
// dK/dV pass (k_bwd_dkdv): workgroup = one 128-key tile; wave w owns keys
// 32w..32w+31 for every query head of the GQA group.  Per 64-row query step:
// S = Q K^T and dP = dO V^T (A = Q/dO from LDS, B = K/V in registers), then
// dV += P^T dO and dK += dS^T Q with P / dS straight from the accumulators and
// dO / Q read back with transposing LDS loads.
#include <climits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace isattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D, int PITCH, int ROWS, int NT, bool PERM>
__device__ __forceinline__ void stage(uint16_t* dst, const uint16_t* src, int64_t row_stride, int row0,
                                      int limit, int tid) {
    TileStager<D, PITCH, ROWS, NT, PERM> t;
    t.load(src, row_stride, row0, limit, tid);
    t.store(dst, tid);
}

// B operand (k = 8 consecutive tile rows, n = 32 columns) of a 32x32x16 MFMA
// from a swap23-staged row-major tile: logical rows 16*cc + 8*h + 0..7 of the
// 32-row group starting at `row32`, columns col0 + (lane % 32).
__device__ __forceinline__ bf16x8_t b_operand_tr(const uint16_t* tile, int pitch, int row32, int cc, int col0,
                                                 int lane) {
    const int L = lane & 15;
    const int g = lane >> 4;
    const int h = g >> 1;
    const int row = row32 + 16 * cc + 4 * h + (L >> 2);
    const int col = col0 + 16 * (g & 1) + 4 * (L & 3);
    const u32x2_t lo = lds_read_tr16(tile + row * pitch + col);
    const u32x2_t hi = lds_read_tr16(tile + (row + 8) * pitch + col);
    const u32x4_t v = {lo[0], lo[1], hi[0], hi[1]};
    return as_bf16x8(v);
}

// Pipeline shared by both passes (three LDS stages, one barrier per step):
//   phase 1  finish the previous step's output GEMM from its stage (the only
//            transposing LDS reads; the compiler's wait for outstanding
//            direct-to-LDS loads lands here, on the loads of this step)
//   barrier  this step's stage is complete in every wave
//   phase 2  issue the direct-to-LDS loads of the next step into the third stage
//   phase 3  S / dP of this step (ds_read_b128 operands, double-buffered)
//   phase 4  P and dS in registers, kept packed for the next step's phase 1

// 16-byte global row chunk as an MFMA operand (resident operands are read once
// per workgroup straight from HBM).
__device__ __forceinline__ bf16x8_t gload_operand(const uint16_t* p) { return as_bf16x8(gload128(p)); }

// ---------------------------------------------------------------------------
// dQ pass
// ---------------------------------------------------------------------------
template <int DQK, int DV, int WR>
struct DqCfg {
    static constexpr int BM = 128;                 // query rows per workgroup
    static constexpr int BN = 32;                  // keys per step
    static constexpr int NW = BM / WR;
    static constexpr int NT = 64 * NW;
    static constexpr int QT = WR / 32;             // 32-row query tiles per wave
    static constexpr int STAGE = BN * (DQK + DV);  // elements per K/V stage
    static constexpr int LDS_BYTES = 3 * STAGE * 2;
    static constexpr int NCQ = DQK / 16;
    static constexpr int NCV = DV / 16;
    static constexpr int NDT = DQK / 32;
};

template <int DQK, int DV, int WR>
__global__ __launch_bounds__(64 * (128 / WR), 1) void k_bwd_dq(BwdArgs a) {
    using C = DqCfg<DQK, DV, WR>;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31, h2 = lane >> 5;

    const int BH = a.B * a.Hq;
    const int id = blockIdx.x;
    const int qb = a.n_qb - 1 - id / BH;          // longest rows first under a causal mask
    const int bh = id - (id / BH) * BH;
    const int b = bh / a.Hq;
    const int h = bh - b * a.Hq;
    const int hk = h / a.G;
    const int m_base = qb * C::BM;
    const int last_row = min(m_base + C::BM - 1, a.Sq - 1);
    const int shift = a.Sk - a.Sq;
    const int diag = last_row + shift;

    int kb_count;
    const int32_t* kb_list = nullptr;
    if (a.mask_kind == 1) {
        const int hm = h * a.Hm / a.Hq;
        const int r = (b * a.Hm + hm) * a.n_qb + qb;
        const int beg = a.q2k_ptr[r];
        kb_count = a.q2k_ptr[r + 1] - beg;
        kb_list = a.q2k_col + beg;
    } else {
        kb_count = a.n_kb;
        if (a.causal) kb_count = diag < 0 ? 0 : min(a.n_kb, diag / kBlock + 1);
    }
    constexpr int SUB = kBlock / C::BN;            // steps per key block
    const int T = kb_count * SUB;
    auto step_n0 = [&](int t) -> int {             // key offset of step t, -1 if nothing visible
        const int kb = kb_list ? kb_list[t / SUB] : t / SUB;
        const int n0 = kb * kBlock + (t % SUB) * C::BN;
        const bool ok = kb >= 0 && kb < a.n_kb && n0 < a.Sk && (!a.causal || n0 <= diag);
        return ok ? n0 : -1;
    };
    auto next_step = [&](int t, int* n0) -> int {
        for (++t; t < T; ++t) {
            *n0 = step_n0(t);
            if (*n0 >= 0) break;
        }
        return t;
    };

    // ---- resident operands: this wave's Q / dO rows (B operands), LSE, delta
    const int wrow = w * WR;
    bf16x8_t qB[C::QT][C::NCQ], doB[C::QT][C::NCV];
    float lse2[C::QT], dlt[C::QT];
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt) {
        const int qrow = m_base + wrow + 32 * qt + l32;
        const bool in = qrow < a.Sq;
        const uint16_t* qr = a.q + b * a.q_sb + h * a.q_sh + int64_t(in ? qrow : 0) * a.q_ss + 8 * h2;
        const uint16_t* dr = a.dO + b * a.do_sb + h * a.do_sh + int64_t(in ? qrow : 0) * a.do_ss + 8 * h2;
#pragma unroll
        for (int c = 0; c < C::NCQ; ++c) qB[qt][c] = in ? gload_operand(qr + 16 * c) : bf16x8_t{};
#pragma unroll
        for (int c = 0; c < C::NCV; ++c) doB[qt][c] = in ? gload_operand(dr + 16 * c) : bf16x8_t{};
        lse2[qt] = __builtin_inff();
        dlt[qt] = 0.f;
        if (in) {
            const int64_t si = (int64_t(b) * a.Hq + h) * a.Sq + qrow;
            lse2[qt] = a.lse[si] * kLog2e;
            dlt[qt] = a.delta[si];
        }
    }

    f32x16_t dq[C::QT][C::NDT];
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
        for (int t = 0; t < C::NDT; ++t) dq[qt][t] = f32x16_t{};

    const uint16_t* gk = a.k + b * a.k_sb + hk * a.k_sh;
    const uint16_t* gv = a.v + b * a.v_sb + hk * a.v_sh;
    auto issue = [&](int n0, int stage_i) {
        uint16_t* base = lds + stage_i * C::STAGE;
        load_tile_async<DQK, C::BN, C::NW>(base, gk, a.k_ss, n0, a.Sk, w, lane);
        load_tile_async<DV, C::BN, C::NW>(base + C::BN * DQK, gv, a.v_ss, n0, a.Sk, w, lane);
    };
    bf16x8_t dsa[C::QT][2];                        // packed dS of the previous step
    auto dq_update = [&](int stage_i) {
        const uint16_t* sK = lds + stage_i * C::STAGE;
        constexpr int NF = 2 * C::NDT;             // B fragments, f = cc * NDT + dt
        constexpr int PF = NF < 3 ? NF : 3;        // prefetch depth
        bf16x8_t fr[PF + 1];
#pragma unroll
        for (int f = 0; f < PF; ++f) fr[f] = b_operand_tr_swz<DQK>(sK, 0, f / C::NDT, 32 * (f % C::NDT), lane);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (f + PF < NF)
                fr[(f + PF) % (PF + 1)] = b_operand_tr_swz<DQK>(sK, 0, (f + PF) / C::NDT, 32 * ((f + PF) % C::NDT), lane);
            const int cc = f / C::NDT, dt = f % C::NDT;
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt) dq[qt][dt] = mfma32(dsa[qt][cc], fr[f % (PF + 1)], dq[qt][dt]);
        }
    };

    int n0 = -1;
    int t = next_step(-1, &n0);
    if (t < T) issue(n0, 0);
    int sidx = 0;
    bool has_prev = false;
    while (t < T) {
        int n0n = -1;
        const int tn = next_step(t, &n0n);
        const int cur = sidx % 3;
        if (has_prev) dq_update((sidx + 2) % 3);
        wait_vmcnt<0>();
        __syncthreads();
        if (tn < T) issue(n0n, (sidx + 1) % 3);

        const uint16_t* sK = lds + cur * C::STAGE;
        const uint16_t* sV = sK + C::BN * DQK;
        f32x16_t st[C::QT], dpt[C::QT];
#pragma unroll
        for (int qt = 0; qt < C::QT; ++qt) {
            st[qt] = f32x16_t{};
            dpt[qt] = f32x16_t{};
        }
        {
            constexpr int PF = 2;                  // prefetch depth (chunks)
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
            }
        }

        // P, dS; accumulator register i holds key n0 + 16*(i/8) + 8*h2 + i%8
        const bool need_mask = (n0 + C::BN > a.Sk) || (a.causal && n0 + C::BN - 1 > m_base + shift);
        if (need_mask) {
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt) {
                const int qrow = m_base + wrow + 32 * qt + l32;
                const int nmax = min(a.Sk - 1, a.causal ? qrow + shift : a.Sk - 1);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int n = n0 + 16 * (i >> 3) + 8 * h2 + (i & 7);
                    float p = fast_exp2(st[qt][i] * a.scale_log2 - lse2[qt]);
                    p = n <= nmax ? p : 0.f;
                    dpt[qt][i] = p * (dpt[qt][i] - dlt[qt]);
                }
            }
        } else {
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = fast_exp2(st[qt][i] * a.scale_log2 - lse2[qt]);
                    dpt[qt][i] = p * (dpt[qt][i] - dlt[qt]);
                }
        }
#pragma unroll
        for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                u32x4_t pk;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    pk[j] = pack_bf16x2(dpt[qt][8 * cc + 2 * j], dpt[qt][8 * cc + 2 * j + 1]);
                dsa[qt][cc] = as_bf16x8(pk);
            }
        has_prev = true;
        ++sidx;
        t = tn;
        n0 = n0n;
    }
    if (has_prev) dq_update((sidx + 2) % 3);

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
// ---------------------------------------------------------------------------
template <int DQK, int DV>
struct DkvCfg {
    static constexpr int BN = 128;                 // keys per workgroup
    static constexpr int BM = 64;                  // query rows per step
    static constexpr int NW = 4;
    static constexpr int NT = 256;
    static constexpr int TILE = BM * (DQK + DV);   // Q and dO tiles of one stage
    static constexpr int STAGE = TILE + 4 * BM;    // + float lse2[BM], delta[BM]
    static constexpr int LDS_BYTES = 3 * STAGE * 2;
    static constexpr int NCQ = DQK / 16;
    static constexpr int NCV = DV / 16;
    static constexpr int NDK = DQK / 32;
    static constexpr int NDV = DV / 32;
    static_assert((STAGE * 2) % 16 == 0 && (TILE * 2) % 16 == 0, "stage alignment");
};

template <int DQK, int DV>
__global__ __launch_bounds__(256, 1) void k_bwd_dkdv(BwdArgs a) {
    using C = DkvCfg<DQK, DV>;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31, h2 = lane >> 5;

    const int BH = a.B * a.Hk;
    const int id = blockIdx.x;
    const int kb = id / BH;                        // longest key columns first under a causal mask
    const int bh = id - kb * BH;
    const int b = bh / a.Hk;
    const int hk = bh - b * a.Hk;
    const int n_base = kb * C::BN;
    const int shift = a.Sk - a.Sq;

    // ---- resident operands: K / V rows of this wave's keys (B operands)
    const int nk = 32 * w + l32;
    const int key = n_base + nk;
    const bool key_in = key < a.Sk;
    bf16x8_t kB[C::NCQ], vB[C::NCV];
    {
        const uint16_t* kr = a.k + b * a.k_sb + hk * a.k_sh + int64_t(key_in ? key : 0) * a.k_ss + 8 * h2;
        const uint16_t* vr = a.v + b * a.v_sb + hk * a.v_sh + int64_t(key_in ? key : 0) * a.v_ss + 8 * h2;
#pragma unroll
        for (int c = 0; c < C::NCQ; ++c) kB[c] = key_in ? gload_operand(kr + 16 * c) : bf16x8_t{};
#pragma unroll
        for (int c = 0; c < C::NCV; ++c) vB[c] = key_in ? gload_operand(vr + 16 * c) : bf16x8_t{};
    }

    f32x16_t dk[C::NDK], dv[C::NDV];
#pragma unroll
    for (int t = 0; t < C::NDK; ++t) dk[t] = f32x16_t{};
#pragma unroll
    for (int t = 0; t < C::NDV; ++t) dv[t] = f32x16_t{};

    const bool tile_ragged = n_base + C::BN > a.Sk;
    // query row q sees this lane's key iff the key is in range and (not causal or key <= q + shift)
    const int qmin = key_in ? (a.causal ? key - shift : INT_MIN) : INT_MAX;

    // ---- step iterator over (query head of the group, kept query block, 64-row half)
    int gi = 0, it = 0, half = 0, qb_count = 0, qb_first = 0;
    const int32_t* qb_list = nullptr;
    auto load_head = [&]() {
        const int hq = hk * a.G + gi;
        qb_list = nullptr;
        qb_first = 0;
        if (a.mask_kind == 1) {
            const int hm = hq * a.Hm / a.Hq;
            const int r = (b * a.Hm + hm) * a.n_kb + kb;
            const int beg = a.k2q_ptr[r];
            qb_count = a.k2q_ptr[r + 1] - beg;
            qb_list = a.k2q_col + beg;
        } else {
            if (a.causal) {
                const int first_row = n_base - shift;
                qb_first = first_row <= 0 ? 0 : first_row / kBlock;
            }
            qb_count = a.n_qb - qb_first;
        }
    };
    auto cur_m0 = [&]() -> int {                   // m0 of (gi, it, half), -1 if no row sees the tile
        const int qb = qb_list ? qb_list[it] : qb_first + it;
        const int m0 = qb * kBlock + half * C::BM;
        if (qb < 0 || qb >= a.n_qb || m0 >= a.Sq) return -1;
        const int mlast = min(m0 + C::BM - 1, a.Sq - 1);
        if (a.causal && mlast + shift < n_base) return -1;
        return m0;
    };
    auto advance = [&](int* m0) -> bool {          // to the next valid step; false at the end
        for (;;) {
            if (++half == kBlock / C::BM) {
                half = 0;
                ++it;
            }
            while (it >= qb_count) {
                if (++gi >= a.G) return false;
                it = 0;
                half = 0;
                load_head();
            }
            *m0 = cur_m0();
            if (*m0 >= 0) return true;
        }
    };

    const int64_t srow_g = int64_t(b) * a.Hq;
    float statv = 0.f;                             // this thread's LSE*log2e or delta of a staged row
    auto issue = [&](int hq, int m0, int stage_i) {
        uint16_t* base = lds + stage_i * C::STAGE;
        load_tile_async<DQK, C::BM, C::NW>(base, a.q + b * a.q_sb + hq * a.q_sh, a.q_ss, m0, a.Sq, w, lane);
        load_tile_async<DV, C::BM, C::NW>(base + C::BM * DQK, a.dO + b * a.do_sb + hq * a.do_sh, a.do_ss, m0,
                                          a.Sq, w, lane);
        if (tid < 2 * C::BM) {
            const int row = m0 + (tid & (C::BM - 1));
            const int64_t si = (srow_g + hq) * a.Sq + row;
            if (tid < C::BM) statv = row < a.Sq ? a.lse[si] * kLog2e : __builtin_inff();
            else statv = row < a.Sq ? a.delta[si] : 0.f;
        }
    };
    auto store_stats = [&](int stage_i) {
        if (tid < 2 * C::BM) {
            float* st = reinterpret_cast<float*>(lds + stage_i * C::STAGE + C::TILE);
            st[(tid & ~(C::BM - 1)) + swap23(tid & (C::BM - 1))] = statv;
        }
    };
    bf16x8_t pa[2][2], sa[2][2];                   // packed P / dS of the previous step
    auto dkv_update = [&](int stage_i) {
        const uint16_t* sQ = lds + stage_i * C::STAGE;
        const uint16_t* sdO = sQ + C::BM * DQK;
        // MFMA f: group g = f / (NDV + NDK) = (mt, cc); within it dV tiles first, then dK tiles
        constexpr int PG = C::NDV + C::NDK;
        constexpr int NF = 4 * PG;
        constexpr int PF = 4;                      // prefetch depth (fragments)
        auto frag = [&](int f) -> bf16x8_t {
            const int g = f / PG, j = f % PG;
            const int mt = g >> 1, cc = g & 1;
            return j < C::NDV ? b_operand_tr_swz<DV>(sdO, 32 * mt, cc, 32 * j, lane)
                              : b_operand_tr_swz<DQK>(sQ, 32 * mt, cc, 32 * (j - C::NDV), lane);
        };
        bf16x8_t fr[PF + 1];
#pragma unroll
        for (int f = 0; f < PF; ++f) fr[f] = frag(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (f + PF < NF) fr[(f + PF) % (PF + 1)] = frag(f + PF);
            const int g = f / PG, j = f % PG;
            const int mt = g >> 1, cc = g & 1;
            if (j < C::NDV) dv[j] = mfma32(pa[mt][cc], fr[f % (PF + 1)], dv[j]);
            else dk[j - C::NDV] = mfma32(sa[mt][cc], fr[f % (PF + 1)], dk[j - C::NDV]);
        }
    };

    load_head();
    int m0 = -1;
    bool have = qb_count > 0;
    if (have) {
        m0 = cur_m0();
        if (m0 < 0) have = advance(&m0);
    }
    if (have) issue(hk * a.G + gi, m0, 0);
    int sidx = 0;
    bool has_prev = false;
    while (have) {
        int m0n = -1;
        const bool more = advance(&m0n);
        const int next_h = hk * a.G + gi;
        const int cur = sidx % 3;
        if (has_prev) dkv_update((sidx + 2) % 3);
        wait_vmcnt<0>();
        store_stats(cur);
        __syncthreads();
        if (more) issue(next_h, m0n, (sidx + 1) % 3);

        const uint16_t* sQ = lds + cur * C::STAGE;
        const uint16_t* sdO = sQ + C::BM * DQK;
        const float* sL = reinterpret_cast<const float*>(lds + cur * C::STAGE + C::TILE);
        const float* sD = sL + C::BM;

        f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
        f32x16_t dp[2] = {f32x16_t{}, f32x16_t{}};
        {
            constexpr int PF = 2;                  // prefetch depth (chunks)
            bf16x8_t qa[PF + 1][2], oa[PF + 1][2];
#pragma unroll
            for (int c = 0; c < PF; ++c)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    qa[c][mt] = row_operand_swz<DQK>(sQ, 32 * mt + l32, 16 * c + 8 * h2);
                    if (c < C::NCV) oa[c][mt] = row_operand_swz<DV>(sdO, 32 * mt + l32, 16 * c + 8 * h2);
                }
#pragma unroll
            for (int c = 0; c < C::NCQ; ++c) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    if (c + PF < C::NCQ)
                        qa[(c + PF) % (PF + 1)][mt] = row_operand_swz<DQK>(sQ, 32 * mt + l32, 16 * (c + PF) + 8 * h2);
                    if (c + PF < C::NCV)
                        oa[(c + PF) % (PF + 1)][mt] = row_operand_swz<DV>(sdO, 32 * mt + l32, 16 * (c + PF) + 8 * h2);
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) s[mt] = mfma32(qa[c % (PF + 1)][mt], kB[c], s[mt]);
                if (c < C::NCV) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) dp[mt] = mfma32(oa[c % (PF + 1)][mt], vB[c], dp[mt]);
                }
            }
        }

        // LSE / delta of this lane's accumulator rows: LDS rows 32*mt + 8*g + 4*h2 + 0..3
        float4 l4[2][4], d4[2][4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                l4[mt][g] = *reinterpret_cast<const float4*>(sL + 32 * mt + 8 * g + 4 * h2);
                d4[mt][g] = *reinterpret_cast<const float4*>(sD + 32 * mt + 8 * g + 4 * h2);
            }
        const bool need_mask = tile_ragged || (a.causal && n_base + C::BN - 1 > m0 + shift);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float4 lv = l4[mt][i >> 2];
                const float4 dv4 = d4[mt][i >> 2];
                const float lse = (i & 3) == 0 ? lv.x : (i & 3) == 1 ? lv.y : (i & 3) == 2 ? lv.z : lv.w;
                const float dl = (i & 3) == 0 ? dv4.x : (i & 3) == 1 ? dv4.y : (i & 3) == 2 ? dv4.z : dv4.w;
                float p = fast_exp2(s[mt][i] * a.scale_log2 - lse);
                if (need_mask) {
                    const int qrow = m0 + 32 * mt + 16 * (i >> 3) + 8 * h2 + (i & 7);
                    p = qrow >= qmin ? p : 0.f;
                }
                dp[mt][i] = p * (dp[mt][i] - dl);
                s[mt][i] = p;
            }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                u32x4_t pp, pd;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pp[j] = pack_bf16x2(s[mt][8 * cc + 2 * j], s[mt][8 * cc + 2 * j + 1]);
                    pd[j] = pack_bf16x2(dp[mt][8 * cc + 2 * j], dp[mt][8 * cc + 2 * j + 1]);
                }
                pa[mt][cc] = as_bf16x8(pp);
                sa[mt][cc] = as_bf16x8(pd);
            }
        has_prev = true;
        ++sidx;
        have = more;
        m0 = m0n;
    }
    if (has_prev) dkv_update((sidx + 2) % 3);

    uint16_t* gdk = a.dk + b * a.dk_sb + hk * a.dk_sh;
    uint16_t* gdv = a.dv + b * a.dv_sb + hk * a.dv_sh;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int n = n_base + 32 * w + 8 * (i >> 2) + 4 * h2 + (i & 3);
        if (n < a.Sk) {
#pragma unroll
            for (int dt = 0; dt < C::NDK; ++dt) gdk[n * a.dk_ss + 32 * dt + l32] = to_bf16(dk[dt][i] * a.scale);
#pragma unroll
            for (int dt = 0; dt < C::NDV; ++dt) gdv[n * a.dv_ss + 32 * dt + l32] = to_bf16(dv[dt][i]);
        }
    }
}

template <int DQK, int DV, int WR>
hipError_t launch_dq_t(const BwdArgs& a, hipStream_t s) {
    using C = DqCfg<DQK, DV, WR>;
    const int64_t grid = int64_t(a.n_qb) * a.B * a.Hq;
    if (grid == 0) return hipSuccess;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k_bwd_dq<DQK, DV, WR>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       C::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((k_bwd_dq<DQK, DV, WR>), dim3(unsigned(grid)), dim3(C::NT), C::LDS_BYTES, s, a);
    return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t s) {
    using C = DkvCfg<DQK, DV>;
    const int64_t grid = int64_t(a.n_kb) * a.B * a.Hk;
    if (grid == 0) return hipSuccess;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k_bwd_dkdv<DQK, DV>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       C::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((k_bwd_dkdv<DQK, DV>), dim3(unsigned(grid)), dim3(C::NT), C::LDS_BYTES, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_split_dkdv(const BwdArgs& a, hipStream_t s) {
    if (a.Dqk == 64 && a.Dv == 64) return launch_dkdv_t<64, 64>(a, s);
    if (a.Dqk == 128 && a.Dv == 128) return launch_dkdv_t<128, 128>(a, s);
    if (a.Dqk == 192 && a.Dv == 128) return launch_dkdv_t<192, 128>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_split_dq(const BwdArgs& a, hipStream_t s) {
    if (a.Dqk == 64 && a.Dv == 64) return launch_dq_t<64, 64, 64>(a, s);
    if (a.Dqk == 128 && a.Dv == 128) return launch_dq_t<128, 128, 64>(a, s);
    if (a.Dqk == 192 && a.Dv == 128) return launch_dq_t<192, 128, 32>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace isattn
