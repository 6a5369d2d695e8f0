// Attention forward on the same mask descriptor as the backward: O and the
// natural-log LSE of the scaled scores over the kept keys (MagiAttention
// PR #334, Summary: the forward statistics the backward recomputes P from;
// the online-rescaling recipe of the nvfp4-megamoe-kernel log's attention
// notes).
//
// Workgroup = one 128-row query tile of one query head; each of the 4 waves
// owns 32 query rows whose Q rows stay in registers.  Per 32-key step of a
// kept key block:
//   S^T = K Q^T      (A = K rows from LDS, B = Q resident; lane = query row,
//                     accumulator register i = key 16*(i/8) + 8*(lane/32) + i%8
//                     with K staged at LDS row swap23(r))
//   online softmax   per lane: the running maximum m (log2 units) moves only
//                     when a step's maximum exceeds it by more than kRescale,
//                     so the O accumulators are rescaled rarely; P values up to
//                     2^kRescale are exact in fp32 and representable in bf16
//   O^T += V^T P^T   (A = V^T by transposing LDS reads, B = P^T packed bf16
//                     straight from the S^T accumulator; lane = query row)
// and at the end O = O^T / l and LSE = ln 2 * (m + log2 l), or +inf and O = 0
// for a row with no kept key.  K/V tiles go through a 4-stage LDS ring filled
// by direct global->LDS loads issued two steps ahead.
#include <climits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "key_steps.hpp"

namespace isattn {
namespace {

constexpr float kRescale = 8.f;   // log2 headroom of the running maximum
constexpr float kLn2 = 0.6931471805599453f;

template <int DQK, int DV, bool TOK>
struct FwdCfg {
    static constexpr int BM = 128;                 // query rows per workgroup
    static constexpr int BN = 32;                  // keys per step
    static constexpr int NW = 4;                   // 32 query rows per wave
    static constexpr int NT = 64 * NW;
    static constexpr int K_BYTES = BN * DQK * 2;
    static constexpr int V_BYTES = BN * DV * 2;
    static constexpr int TILE_BYTES = K_BYTES + V_BYTES;
    // token-exact masks: each wave's 32 rows' bit words of the step (64 lanes x 4 B)
    static constexpr int TK_BYTES = TOK ? NW * 256 : 0;
    static constexpr int STAGE_BYTES = TILE_BYTES + TK_BYTES;
    static constexpr int NS = 4;                   // LDS ring stages (loads run two steps ahead)
    static constexpr int LDS_BYTES = NS * STAGE_BYTES;
    static constexpr int NKI = K_BYTES / 1024;     // 1 KiB loads per K tile
    static constexpr int NI = TILE_BYTES / 1024;   // 1 KiB loads per step
    static constexpr int KMAX = NI / NW;           // tile loads per wave per step
    static constexpr int NL = KMAX + (TOK ? 1 : 0);   // loads per wave per step
    static constexpr int NCQ = DQK / 16;
    static constexpr int NDT = DV / 32;            // O^T row tiles (32 columns of O each)
    static_assert(NI % NW == 0 && K_BYTES % 1024 == 0, "tiles split into whole wave loads");
    static_assert(NL <= NCQ, "loads must fit between the S MFMAs");
};

template <int DQK, int DV, bool VL, bool TOK>
__global__ __launch_bounds__(256, 2) void k_attn_fwd(FwdArgs a) {
    using C = FwdCfg<DQK, DV, TOK>;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h2 = lane >> 5;

    // items (b, h, query block), head-major; within a head the longest rows
    // (most visible keys under a causal mask) first
    const int item = xcd_item(blockIdx.x, a.n_qb * a.B * a.Hq);
    if (item < 0) return;
    const int bh = item / a.n_qb;
    const int qb = a.n_qb - 1 - (item - bh * a.n_qb);
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

    // ---- resident operand: this wave's Q rows (B operand of S^T = K Q^T)
    const int qrow = m_base + 32 * w + l32;
    bf16x8_t qB[C::NCQ];
    {
        const bool in = qrow < a.Sq;
        const uint16_t* qr = a.q + b * a.q_sb + h * a.q_sh + int64_t(in ? qrow : 0) * a.q_ss + 8 * h2;
#pragma unroll
        for (int c = 0; c < C::NCQ; ++c) qB[c] = in ? gload_operand(qr + 16 * c) : bf16x8_t{};
    }
    f32x16_t o[C::NDT];
#pragma unroll
    for (int t = 0; t < C::NDT; ++t) o[t] = f32x16_t{};
    float m_run = -__builtin_inff();              // running maximum (log2 units), same in both lane halves
    float l_run = 0.f;                            // this lane's half of the row sum, relative to m_run

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
    // loads its row's word (rows 32 w + L % 32) for the step's 32 keys
    const uint32_t* tslots = nullptr;
    const uint32_t tk_off = uint32_t(16 * (32 * w + l32));
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

    // One step: S^T of stage s (loads for two steps ahead go out between the
    // MFMAs), the online softmax, O^T += V^T P^T.
    auto step = [&](int s, int n0) {
        const uint16_t* sK = lds + s * (C::STAGE_BYTES / 2);
        const uint16_t* sV = sK + C::K_BYTES / 2;
        uint32_t tw = ~0u;
        if constexpr (TOK) tw = *reinterpret_cast<const uint32_t*>(sK + (C::TILE_BYTES + 256 * w + 4 * l32) / 2);
        f32x16_t st = f32x16_t{};
        {
            constexpr int PF = 2;                  // K rows read this many chunks ahead
            bf16x8_t ka[PF + 1];
#pragma unroll
            for (int c = 0; c < PF; ++c) ka[c] = row_operand_swz<DQK>(sK, l32, 16 * c + 8 * h2);
#pragma unroll
            for (int c = 0; c < C::NCQ; ++c) {
                if (c + PF < C::NCQ) ka[(c + PF) % (PF + 1)] = row_operand_swz<DQK>(sK, l32, 16 * (c + PF) + 8 * h2);
                st = mfma32(ka[c % (PF + 1)], qB[c], st);
                if (c < C::NL) fire(c);
            }
        }
        // scores in log2 units; keys past Sk or (causal) past the row's last
        // visible key are -inf
        float sv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[i] = st[i] * a.scale_log2;
        if ((n0 + C::BN > a.Sk) || (a.causal && n0 + C::BN - 1 > m_base + shift)) {
            const int rel = min(a.Sk - 1, a.causal ? qrow + shift : a.Sk - 1) - n0 - 8 * h2;
#pragma unroll
            for (int i = 0; i < 16; ++i) sv[i] = 16 * (i >> 3) + (i & 7) <= rel ? sv[i] : -__builtin_inff();
        }
        if constexpr (TOK) {                       // keys the row did not select
            const uint32_t mine = tw >> (8 * h2);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (((mine >> (16 * (i >> 3) + (i & 7))) & 1u) == 0) sv[i] = -__builtin_inff();
        }
        float mx = sv[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));    // the row's other 16 keys
        // move the running maximum only when it grows by more than kRescale
        if (mx > m_run + kRescale) {
            const float alpha = fast_exp2(m_run - mx);   // 0 while m_run is -inf
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < C::NDT; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
            m_run = mx;
        }
        const float mref = m_run == -__builtin_inff() ? 0.f : m_run;
        u32x4_t pk[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float p0 = fast_exp2(sv[8 * cc + 2 * j] - mref);
                const float p1 = fast_exp2(sv[8 * cc + 2 * j + 1] - mref);
                l_run += p0 + p1;
                pk[cc][j] = pack_bf16x2(p0, p1);
            }
        // O^T += V^T P^T: A = V^T fragment (column tile dt, key chunk cc)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
                o[dt] = mfma32(b_operand_tr_swz<DV>(sV, 0, cc, 32 * dt, lane), as_bf16x8(pk[cc]), o[dt]);
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
        step(0, n0);
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
            step(t % C::NS, n0);
            have1 = have2;
            n1 = n2;
            have2 = have3;
            n2 = n3;
        }
        wait_vmcnt<0>();                           // no load may land in LDS after the workgroup ends
    }

    // ---- O = O^T / l (lane = query row; register i of tile dt = column
    // 32*dt + 8*(i/4) + 4*(lane/32) + i%4) and LSE
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (qrow < a.Sq) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* orow = a.o + b * a.o_sb + h * a.o_sh + int64_t(qrow) * a.o_ss;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2_t pkd;
                pkd[0] = pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv);
                pkd[1] = pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
                *reinterpret_cast<u32x2_t*>(orow + 32 * dt + 8 * g + 4 * h2) = pkd;
            }
        if (h2 == 0)
            a.lse[(int64_t(b) * a.Hq + h) * a.lse_ld + qrow] =
                l_tot > 0.f ? kLn2 * (m_run + __builtin_amdgcn_logf(l_tot)) : __builtin_inff();
    }
}

template <int DQK, int DV, bool VL, bool TOK>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
    using C = FwdCfg<DQK, DV, TOK>;
    const int64_t items = int64_t(a.n_qb) * a.B * a.Hq;
    if (items == 0) return hipSuccess;
    const int64_t grid = int64_t(kXcds) * xcd_items_per(int(items));
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k_attn_fwd<DQK, DV, VL, TOK>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       C::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((k_attn_fwd<DQK, DV, VL, TOK>), dim3(unsigned(grid)), dim3(C::NT), C::LDS_BYTES, s, a);
    return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t s) {
    if (a.tok != nullptr)
        return a.cu_q != nullptr ? launch_fwd_t<DQK, DV, true, true>(a, s) : launch_fwd_t<DQK, DV, false, true>(a, s);
    return a.cu_q != nullptr ? launch_fwd_t<DQK, DV, true, false>(a, s) : launch_fwd_t<DQK, DV, false, false>(a, s);
}

}  // namespace

hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t s) {
    if (a.Dqk == 64 && a.Dv == 64) return launch_fwd_d<64, 64>(a, s);
    if (a.Dqk == 128 && a.Dv == 128) return launch_fwd_d<128, 128>(a, s);
    if (a.Dqk == 192 && a.Dv == 128) return launch_fwd_d<192, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace isattn
