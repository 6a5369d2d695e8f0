// LoopK attention backward: outer loop over query tiles, inner loop over the
// kept key tiles (MagiAttention PR #334, Summary and Core changes item 1: dQ
// accumulates on chip and is stored once; dK/dV partials of every key step
// are reduced into fp32 global accumulators; Core changes item 2: sparse
// iteration over each query block's list of key blocks).
//
// One workgroup = 4 waves = one 128-row query tile of one (batch, head).
// Each inner step stages 64 keys of K (row-major and transposed) and V in LDS.
// Per step and wave (wave w owns queries 32w..32w+31 of the tile):
//
//   S^T  = K Q^T      [64 keys x 32 q]  32x32x16 MFMA, A = K (LDS), B = Q (regs)
//   dP^T = V dO^T     [64 keys x 32 q]  same, B = dO (regs)
//   P    = exp2(S^T * scale*log2e - LSE*log2e),  dS = P * (dP - delta)
//   dQ  += dS K       [32 q x Dqk]      A = dS straight from the S^T
//                                       accumulator registers (the accumulator's
//                                       column = this lane's query = the A row)
//   P^T, dS^T -> LDS (bf16) so every wave sees all 128 queries, then
//   dV_part = P^T dO  [64 keys x Dv/4]  16x16x32 MFMA, A = P^T (LDS), B = dO (regs)
//   dK_part = dS^T Q  [64 keys x Dqk/4] A = dS^T (LDS), B = Q (regs)
//   fp32 atomic add of dK_part / dV_part (hardware global_atomic_add_f32).
//
// The k-slot order of the register-sourced A operand of dQ is the
// accumulator's row interleave (rows 4h..4h+3 and 8+4h..8+4h+3 of each
// 16-row chunk for lane half h); the matching B operand is read from the
// transposed K copy as two 8-byte runs.
#include "device_common.hpp"
#include "kernels.hpp"

namespace isattn {
namespace {


template <int DQK, int DV>
struct LoopKCfg {
    static constexpr int BM = 128;                 // query rows per workgroup
    static constexpr int BN = 64;                  // keys per inner step
    static constexpr int NT = 256;                 // 4 waves
    static constexpr int PK = DQK + 8;             // sK row pitch (elements)
    static constexpr int PKT = BN + 4;             // sKt row pitch
    static constexpr int PV = DV + 8;
    static constexpr int PP = BM + 8;              // sP / sdS row pitch
    static constexpr int OFF_K = 0;
    static constexpr int OFF_KT = OFF_K + BN * PK;
    static constexpr int OFF_V = OFF_KT + DQK * PKT;
    static constexpr int OFF_P = OFF_V + BN * PV;
    static constexpr int OFF_DS = OFF_P + BN * PP;
    static constexpr int END_LOOP = OFF_DS + BN * PP;
    static constexpr int PQ = DQK + 8;             // prologue staging pitches
    static constexpr int PDO = DV + 8;
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_DO = BM * PQ;
    static constexpr int END_PRO = OFF_DO + BM * PDO;
    static constexpr int LDS_ELEMS = END_LOOP > END_PRO ? END_LOOP : END_PRO;
    static constexpr int LDS_BYTES = LDS_ELEMS * 2;
    static constexpr int NCQ = DQK / 16;           // 16-wide k chunks over Dqk
    static constexpr int NCV = DV / 16;
    static constexpr int NDT = DQK / 32;           // dQ accumulator tiles
    static constexpr int WQK = DQK / 4;            // dK d-slice per wave
    static constexpr int WV = DV / 4;              // dV d-slice per wave
    static constexpr int NTK = WQK / 16;
    static constexpr int NTV = WV / 16;
    static_assert(WQK % 16 == 0 && WV % 16 == 0, "head dims must split into 16-wide tiles per wave");
};

// Rows [row0, row0 + ROWS) of a [seq, dim] slice into LDS (pitch PITCH), zeros past `limit`.
// Rows [row0, row0 + ROWS) of a [seq, D] slice into LDS (pitch PITCH), zeros past `limit`.
template <int D, int PITCH, int ROWS, int NT>
__device__ __forceinline__ void stage_rows(uint16_t* dst, const uint16_t* src, int64_t row_stride,
                                           int row0, int limit, int tid) {
    TileStager<D, PITCH, ROWS, NT, false> t;
    t.load(src, row_stride, row0, limit, tid);
    t.store(dst, tid);
}

// 64 keys of K: row-major copy (pitch PK) and transposed copy (pitch PKT).
template <int D, int PK, int PKT, int NT>
__device__ __forceinline__ void stage_k(uint16_t* sK, uint16_t* sKt, const uint16_t* src,
                                        int64_t row_stride, int row0, int limit, int tid) {
    TileStager<D, PK, 64, NT, false> t;
    t.load(src, row_stride, row0, limit, tid);
    t.store(sK, tid);
    t.template store_t<PKT>(sKt, tid);
}

template <int DQK, int DV>
__global__ __launch_bounds__(256, 1) void k_bwd_loopk(BwdArgs a) {
    using C = LoopKCfg<DQK, DV>;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31, h2 = lane >> 5;   // 32x32 layout: column, lane half
    const int l16 = lane & 15, g4 = lane >> 4;   // 16x16 layout: column, lane group

    // ---- work item: longest query rows first under a causal mask
    const int BH = a.B * a.Hq;
    const int id = blockIdx.x;
    const int qb = a.n_qb - 1 - id / BH;
    const int bh = id - (id / BH) * BH;
    const int b = bh / a.Hq;
    const int h = bh - b * a.Hq;
    const int hk = h / a.G;
    const int m_base = qb * C::BM;
    const int last_row = min(m_base + C::BM - 1, a.Sq - 1);
    const int shift = a.Sk - a.Sq;               // bottom-right causal: key j visible to row i iff j <= i + shift
    const int diag = last_row + shift;           // largest key visible to any row of the tile

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

    // ---- prologue: Q and dO tiles -> registers
    {
        uint16_t* sQ = lds + C::OFF_Q;
        uint16_t* sdO = lds + C::OFF_DO;
        stage_rows<DQK, C::PQ, C::BM, C::NT>(sQ, a.q + b * a.q_sb + h * a.q_sh, a.q_ss, m_base, a.Sq, tid);
        stage_rows<DV, C::PDO, C::BM, C::NT>(sdO, a.dO + b * a.do_sb + h * a.do_sh, a.do_ss, m_base, a.Sq,
                                             tid);
    }
    __syncthreads();

    const int mq = 32 * w + l32;                 // this lane's query within the tile (32x32 column)
    bf16x8_t qS[C::NCQ], doS[C::NCV];            // B operands of S^T / dP^T
    bf16x8_t qK[C::NTK][4], doV[C::NTV][4];      // B operands of dK / dV (k = query)
    {
        const uint16_t* sQ = lds + C::OFF_Q;
        const uint16_t* sdO = lds + C::OFF_DO;
#pragma unroll
        for (int c = 0; c < C::NCQ; ++c) qS[c] = as_bf16x8(lds_read128(sQ + mq * C::PQ + 16 * c + 8 * h2));
#pragma unroll
        for (int c = 0; c < C::NCV; ++c) doS[c] = as_bf16x8(lds_read128(sdO + mq * C::PDO + 16 * c + 8 * h2));
#pragma unroll
        for (int t = 0; t < C::NTK; ++t) {
            const int d = w * C::WQK + 16 * t + l16;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u32x4_t v;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int m = 32 * c + 8 * g4 + 2 * j;
                    v[j] = uint32_t(sQ[m * C::PQ + d]) | (uint32_t(sQ[(m + 1) * C::PQ + d]) << 16);
                }
                qK[t][c] = as_bf16x8(v);
            }
        }
#pragma unroll
        for (int t = 0; t < C::NTV; ++t) {
            const int d = w * C::WV + 16 * t + l16;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u32x4_t v;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int m = 32 * c + 8 * g4 + 2 * j;
                    v[j] = uint32_t(sdO[m * C::PDO + d]) | (uint32_t(sdO[(m + 1) * C::PDO + d]) << 16);
                }
                doV[t][c] = as_bf16x8(v);
            }
        }
    }
    const int qrow = m_base + mq;
    float lse2 = __builtin_inff();
    float dlt = 0.f;
    if (qrow < a.Sq) {
        const int64_t si = (int64_t(b) * a.Hq + h) * a.Sq + qrow;
        lse2 = a.lse[si] * kLog2e;
        dlt = a.delta[si];
    }
    __syncthreads();

    f32x16_t dq[C::NDT];
#pragma unroll
    for (int t = 0; t < C::NDT; ++t) dq[t] = f32x16_t{};

    uint16_t* sK = lds + C::OFF_K;
    uint16_t* sKt = lds + C::OFF_KT;
    uint16_t* sV = lds + C::OFF_V;
    uint16_t* sP = lds + C::OFF_P;
    uint16_t* sdS = lds + C::OFF_DS;
    const uint16_t* gk = a.k + b * a.k_sb + hk * a.k_sh;
    const uint16_t* gv = a.v + b * a.v_sb + hk * a.v_sh;
    // fp32 accumulators are head-major [B, Hk, Sk, D]: the keys of one step are
    // contiguous, so a step's atomics spread over all L2 channels
    float* gdk = a.acc0 + (int64_t(b) * a.Hk + hk) * a.Sk * DQK;
    float* gdv = a.acc1 + (int64_t(b) * a.Hk + hk) * a.Sk * DV;

    for (int it = 0; it < kb_count; ++it) {
        const int kb = kb_list ? kb_list[it] : it;
        if (kb < 0 || kb >= a.n_kb) continue;      // ignore malformed CSR entries
        if (a.causal && kb * kBlock > diag) continue;
#pragma unroll 1
        for (int half = 0; half < kBlock / C::BN; ++half) {
            const int n0 = kb * kBlock + half * C::BN;
            if (n0 >= a.Sk || (a.causal && n0 > diag)) break;
            stage_k<DQK, C::PK, C::PKT, C::NT>(sK, sKt, gk, a.k_ss, n0, a.Sk, tid);
            stage_rows<DV, C::PV, C::BN, C::NT>(sV, gv, a.v_ss, n0, a.Sk, tid);
            __syncthreads();

            // S^T and dP^T for this wave's 32 queries
            f32x16_t st[2] = {f32x16_t{}, f32x16_t{}};
            f32x16_t dpt[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
            for (int c = 0; c < C::NCQ; ++c) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const bf16x8_t ka = as_bf16x8(lds_read128(sK + (32 * kt + l32) * C::PK + 16 * c + 8 * h2));
                    st[kt] = mfma32(ka, qS[c], st[kt]);
                }
            }
#pragma unroll
            for (int c = 0; c < C::NCV; ++c) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const bf16x8_t va = as_bf16x8(lds_read128(sV + (32 * kt + l32) * C::PV + 16 * c + 8 * h2));
                    dpt[kt] = mfma32(va, doS[c], dpt[kt]);
                }
            }

            // P and dS (registers); P^T, dS^T -> LDS
            const bool need_mask = (n0 + C::BN > a.Sk) || (a.causal && n0 + C::BN - 1 > m_base + shift);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = 32 * kt + 8 * (i >> 2) + 4 * h2 + (i & 3);
                    float p = fast_exp2(st[kt][i] * a.scale_log2 - lse2);
                    if (need_mask) {
                        const int n = n0 + r;
                        const bool ok = n < a.Sk && (!a.causal || n <= qrow + shift);
                        p = ok ? p : 0.f;
                    }
                    const float ds = p * (dpt[kt][i] - dlt);
                    st[kt][i] = p;
                    dpt[kt][i] = ds;
                    sP[r * C::PP + mq] = to_bf16(p);
                    sdS[r * C::PP + mq] = to_bf16(ds);
                }
            }

            // dQ += dS K
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    u32x4_t pk;
#pragma unroll
                    for (int j = 0; j < 4; ++j) pk[j] = pack_bf16x2(dpt[kt][8 * c + 2 * j], dpt[kt][8 * c + 2 * j + 1]);
                    const bf16x8_t dsa = as_bf16x8(pk);
#pragma unroll
                    for (int dt = 0; dt < C::NDT; ++dt) {
                        const uint16_t* src = sKt + (32 * dt + l32) * C::PKT + 32 * kt + 16 * c + 4 * h2;
                        const u32x2_t lo = lds_read64(src);
                        const u32x2_t hi = lds_read64(src + 8);
                        const u32x4_t kv = {lo[0], lo[1], hi[0], hi[1]};
                        dq[dt] = mfma32(dsa, as_bf16x8(kv), dq[dt]);
                    }
                }
            }
            __syncthreads();

            // dV_part = P^T dO and dK_part = dS^T Q on this wave's d-slices; atomics
#pragma unroll
            for (int nt = 0; nt < C::BN / 16; ++nt) {
                bf16x8_t pa[4], sa[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    pa[c] = as_bf16x8(lds_read128(sP + (16 * nt + l16) * C::PP + 32 * c + 8 * g4));
                    sa[c] = as_bf16x8(lds_read128(sdS + (16 * nt + l16) * C::PP + 32 * c + 8 * g4));
                }
                const int key0 = n0 + 16 * nt + 4 * g4;
#pragma unroll
                for (int t = 0; t < C::NTV; ++t) {
                    f32x4_t acc = f32x4_t{};
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc = mfma16(pa[c], doV[t][c], acc);
                    const int d = w * C::WV + 16 * t + l16;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (key0 + i < a.Sk) atomic_add_f32(gdv + int64_t(key0 + i) * DV + d, acc[i]);
                }
#pragma unroll
                for (int t = 0; t < C::NTK; ++t) {
                    f32x4_t acc = f32x4_t{};
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc = mfma16(sa[c], qK[t][c], acc);
                    const int d = w * C::WQK + 16 * t + l16;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (key0 + i < a.Sk) atomic_add_f32(gdk + int64_t(key0 + i) * DQK + d, acc[i]);
                }
            }
            __syncthreads();
        }
    }

    // ---- epilogue: dQ = scale * acc -> bf16, stored once
    uint16_t* gdq = a.dq + b * a.dq_sb + h * a.dq_sh;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = m_base + 32 * w + 8 * (i >> 2) + 4 * h2 + (i & 3);
            if (m < a.Sq) gdq[m * a.dq_ss + 32 * dt + l32] = to_bf16(dq[dt][i] * a.scale);
        }
    }
}

template <int DQK, int DV>
hipError_t launch_t(const BwdArgs& a, hipStream_t s) {
    using C = LoopKCfg<DQK, DV>;
    const int64_t grid = int64_t(a.n_qb) * a.B * a.Hq;
    if (grid == 0) return hipSuccess;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k_bwd_loopk<DQK, DV>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       C::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((k_bwd_loopk<DQK, DV>), dim3(unsigned(grid)), dim3(C::NT), C::LDS_BYTES, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_loopk(const BwdArgs& a, hipStream_t s) {
    if (a.Dqk == 64 && a.Dv == 64) return launch_t<64, 64>(a, s);
    if (a.Dqk == 128 && a.Dv == 128) return launch_t<128, 128>(a, s);
    if (a.Dqk == 192 && a.Dv == 128) return launch_t<192, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace isattn
