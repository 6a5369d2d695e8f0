// dQ pass of SPLIT_DS: dQ = softmax_scale * sum over the kept key blocks of
// dS K, with dS read back from the tiles the dK/dV pass stored instead of
// being recomputed from Q, K, V, dO and the statistics.
//
// The dQ GEMM is the LoopK accumulation of MagiAttention PR #334 (Summary:
// dQ stays on chip over the kept K blocks of a query tile and is stored
// once).  What changes is where dS comes from: the dK/dV pass already forms
// every dS tile (bf16, the MFMA operand precision), and MI355X's 288 GB of
// HBM hold them all for the workloads here, so the second pass streams
// 32 KiB of dS per kept block at HBM speed rather than spending the S and dP
// GEMMs again.
//
// Stored tile (b, h, qb, kb): 128 x 128 bf16 as 32 chunks of 1 KiB; chunk
// 16 p + 4 wr + 2 hh + cc holds keys 32 wr + (0..31) of the key block and
// query rows 64 p + 32 hh + 16 cc + (0..15) of the query block: 16-byte slot
// l + 32 j of the chunk holds key 32 wr + l, rows ... + 8 j + (0..7).  That is
// the register layout of the dK/dV pass's dS waves, so each of their stores
// writes one whole chunk.
//
// Workgroup = one 128-row query tile of one head; wave w owns query rows
// 32 w .. 32 w + 31, i.e. chunk column (p, hh) = (w / 2, w % 2).  A step is 32
// keys (one wr) of a kept key block: the shared K rows (plain row order,
// chunk-swizzled) and each wave's own two dS chunks go through an LDS ring
// filled by direct global->LDS loads two steps ahead (dS with the
// non-temporal hint: each tile is read once, K is reused from L2).  dQ += dS K takes
// both operands by transposing LDS reads (ds_read_b64_tr_b16): dS rows =
// queries with k = keys, K^T columns = head dims with k = the same keys.
// Each dS chunk is copied with a lane permutation that makes those reads
// bank-conflict free (a 32-lane pass then touches each of the 64 banks once).
#include <climits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "key_steps.hpp"

namespace isattn {
namespace {

template <int DQK>
struct DsqCfg {
    static constexpr int BM = 128;                 // query rows per workgroup
    static constexpr int BN = 32;                  // keys per step
    static constexpr int NW = 4;                   // 32 query rows per wave
    static constexpr int NT = 64 * NW;
    static constexpr int K_BYTES = BN * DQK * 2;
    static constexpr int S_BYTES = 2 * 1024;       // one wave's dS of a step: 2 chunks
    static constexpr int STAGE_BYTES = K_BYTES + NW * S_BYTES;
    // ring stages: four make 64 KiB of LDS per workgroup at Dqk = 128, so
    // two workgroups share a CU; that measured 5 % faster than three
    // workgroups of a 3-stage ring (48 KiB each), and deeper rings or one
    // workgroup per CU were slower
    static constexpr int NS = 4;
    static constexpr int AHEAD = 2;                // loads run this many steps ahead
    static_assert(NS >= AHEAD + 1, "a stage is reloaded only after the step that last read it");
    static constexpr int LDS_BYTES = NS * STAGE_BYTES;
    static constexpr int NKI = K_BYTES / 1024;     // 1 KiB loads per K tile
    static constexpr int KL = NKI / NW;            // K loads per wave per step
    static constexpr int NL = KL + 2;              // loads per wave per step (K part, 2 dS chunks)
    static constexpr int NDT = DQK / 32;           // 32-column dQ tiles
    static_assert(NKI % NW == 0, "the K tile splits into whole wave loads");
};

// LDS slot s of a copied dS chunk cc holds the chunk's global slot
// ds_slot(s, cc): bits of s are (l0, l1, j, l2 ^ cc, l3, l4) for global slot
// l + 32 j.
__device__ __forceinline__ int ds_slot(int s, int cc) {
    const int l = (s & 3) | ((((s >> 3) & 1) ^ cc) << 2) | (((s >> 4) & 3) << 3);
    return l + 32 * ((s >> 2) & 1);
}
// LDS byte offset (inside a wave's two copied chunks) of the 8 bytes holding
// key l, query rows 16 cc + 8 j + 4 hf + (0..3).
__device__ __forceinline__ uint32_t ds_lds_off(int l, int cc, int j, int hf) {
    const int s = (l & 3) | (j << 2) | ((((l >> 2) & 1) ^ cc) << 3) | (((l >> 3) & 3) << 4);
    return uint32_t(1024 * cc + 16 * s + 8 * hf);
}

template <int DQK, bool VL>
__global__ __launch_bounds__(256, 2) void k_bwd_dq_ds(BwdArgs a) {
    using C = DsqCfg<DQK>;
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
    if (a.ds_flag != nullptr && *a.ds_flag != 0) return;   // the dS tiles were not stored (overflow)

    // the key blocks the dK/dV pass visited for this query block, and the
    // slots of their dS tiles: block CSR, R * (K->Q position) + the head's
    // place among the R query heads of its mask head (the position map read
    // along with the Q->K list); dense, the head's slot of (qb, kb = 0) + kb
    KeySteps steps;
    init_key_steps(steps, a, b, h, qb, lane);
    const bool csr = a.mask_kind == 1;
    int R = 1, rr = 0;
    int64_t tile0 = 0;
    if (csr) {
        R = a.Hq / a.Hm;
        rr = h - (h * a.Hm / a.Hq) * R;
        steps.aux = a.ds_map + steps.beg;
        steps.aux_n = int(min(int64_t(steps.count), max(int64_t(0), a.ds_map_len - steps.beg)));
    } else {
        tile0 = (int64_t(b) * a.Hq + h) * int64_t(a.ds_T) +
                (VL ? int64_t(qb) * a.n_kb : visible_before(qb, a.Sq, a.Sk, a.n_kb, a.causal != 0));
    }

    f32x16_t dq[C::NDT];
#pragma unroll
    for (int t = 0; t < C::NDT; ++t) dq[t] = f32x16_t{};

    // ---- loads: K part (instruction j = w + NW * kk of the K tile, rows in
    // plain order) and this wave's two dS chunks of the step's key group
    const uint16_t* gk = a.k + b * a.k_sb + hk * a.k_sh;
    const uint32_t lds_base = lds_address(lds);
    auto k_off = [&](int kk, int lim) -> uint32_t {  // tile rows past lim read row lim
        const int e = 512 * (w + C::NW * kk) + 8 * lane;
        const int r = e / DQK;
        const int c = ((e - r * DQK) >> 3) ^ chunk_swz(r, DQK);
        return uint32_t(min(r, lim)) * uint32_t(a.k_ss * 2) + uint32_t(16 * c);
    };
    uint32_t koff[C::KL];
#pragma unroll
    for (int kk = 0; kk < C::KL; ++kk) koff[kk] = k_off(kk, C::BN);
    uint32_t soff[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) soff[cc] = uint32_t(16 * ds_slot(lane, cc));
    const int wchunk = 16 * (w >> 1) + 2 * (w & 1);   // chunk of (p, hh) for wr = 0, cc = 0
    struct Dma {
        const uint16_t* ds;                          // the step's dS tile
        uint32_t dso;                                // byte offset of its chunk pair for this wave
        uint32_t sb;                                 // LDS stage
        uint32_t ko[C::KL];
    } d;
    auto plan = [&](int n0, int s) {
        const int kb = n0 / kBlock;
        const int wr = (n0 - kb * kBlock) / C::BN;
        d.sb = lds_base + uint32_t(s * C::STAGE_BYTES);
        int64_t tile = csr ? int64_t(R) * steps.aux_at() + rr : tile0 + kb;
        tile = min(max(tile, int64_t(0)), int64_t(a.ds_cap) - 1);   // in bounds whatever the mask holds
        d.ds = a.ds + tile * (kBlock * kBlock);
        d.dso = uint32_t((wchunk + 4 * wr) * 1024);
        if (n0 + C::BN <= a.Sk) {
            const uint32_t mk = uint32_t(n0) * uint32_t(a.k_ss * 2);
#pragma unroll
            for (int kk = 0; kk < C::KL; ++kk) d.ko[kk] = koff[kk] + mk;
        } else {                                     // ragged tail: keys past Sk re-read key Sk - 1
            const int nb = min(n0, a.Sk - 1);
            const uint32_t mk = uint32_t(nb) * uint32_t(a.k_ss * 2);
#pragma unroll
            for (int kk = 0; kk < C::KL; ++kk) d.ko[kk] = k_off(kk, a.Sk - 1 - nb) + mk;
        }
    };
    auto restage = [&](int s) { d.sb = lds_base + uint32_t(s * C::STAGE_BYTES); };
    auto fire_all = [&]() {
#pragma unroll
        for (int kk = 0; kk < C::KL; ++kk) dma16(gk, d.ko[kk], d.sb + uint32_t(1024 * (w + C::NW * kk)));
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
            dma16_nt(d.ds, d.dso + uint32_t(1024 * cc) + soff[cc],
                  d.sb + uint32_t(C::K_BYTES + w * C::S_BYTES + 1024 * cc));
    };

    // ---- operand reads (byte offsets from a stage base)
    // A = dS of this wave's rows, k-chunk kc (keys 16 kc .. 16 kc + 15): lane
    // (g = lane / 16, L = lane % 16) reads key 16 kc + 4 (g / 2) + L / 4 (+8
    // for hi) at query rows 16 (g % 2) + 4 (L % 4) + (0..3)
    uint32_t aoff[2][2];
    {
        const int L = lane & 15, g = lane >> 4;
        const int cc = g & 1, j = (L >> 1) & 1, hf = L & 1;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi)
                aoff[kc][hi] = uint32_t(C::K_BYTES + w * C::S_BYTES) +
                               ds_lds_off(16 * kc + 4 * (g >> 1) + (L >> 2) + 8 * hi, cc, j, hf);
    }
    // B = K^T columns 32 dt .. 32 dt + 31, the same keys
    uint32_t boff[C::NDT][2];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) boff[dt][hi] = tr_read_off<DQK>(lane, dt, hi);
    const lds_char* lp = lds_ptr(lds);
    auto tr_pair = [&](const lds_char* p0, const lds_char* p1) {
        const u32x2_t lo = lds_ld_tr16(p0);
        const u32x2_t hi = lds_ld_tr16(p1);
        const u32x4_t v = {lo[0], lo[1], hi[0], hi[1]};
        return as_bf16x8(v);
    };
    auto compute = [&](int s) {
        const lds_char* st = lp + s * C::STAGE_BYTES;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const bf16x8_t av = tr_pair(st + aoff[kc][0], st + aoff[kc][1]);
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) {
                const int ko = 16 * kc * DQK * 2;    // 16 rows on: the swizzle repeats
                const bf16x8_t bv = tr_pair(st + boff[dt][0] + ko, st + boff[dt][1] + ko);
                dq[dt] = mfma32(av, bv, dq[dt]);
            }
        }
    };

    bool more = steps.next_block();                  // steps is at the next step to plan
    if (more) {
        int planned = 0;
        // plan the next step into a stage, or past the end re-load the last
        // planned step's data there (keeps the per-step load count uniform)
        auto plan_next = [&](int stage) {
            if (more) {
                plan(steps.n0, stage);
                ++planned;
                more = steps.next();
            } else {
                restage(stage);
            }
            fire_all();
        };
#pragma unroll
        for (int i = 0; i < C::AHEAD; ++i) plan_next(i);
        for (int t = 0; t < planned; ++t) {
            wait_vmcnt<C::NL * (C::AHEAD - 1)>();    // this wave's loads of step t landed
            __syncthreads();                         // everyone's; stage (t + AHEAD) % NS was last read before step t
            plan_next((t + C::AHEAD) % C::NS);
            compute(t % C::NS);
        }
        wait_vmcnt<0>();                             // no load may land in LDS after the workgroup ends
    }

    uint16_t* gdq = a.dq + b * a.dq_sb + h * a.dq_sh;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = m_base + 32 * w + 8 * (i >> 2) + 4 * h2 + (i & 3);
            if (m < a.Sq) gdq[int64_t(m) * a.dq_ss + 32 * dt + l32] = to_bf16(dq[dt][i] * a.scale);
        }
}

template <int DQK, bool VL>
hipError_t launch_t(const BwdArgs& a, hipStream_t s) {
    using C = DsqCfg<DQK>;
    const int64_t items = int64_t(a.n_qb) * a.B * a.Hq;
    if (items == 0) return hipSuccess;
    const int64_t grid = int64_t(kXcds) * xcd_items_per(int(items));
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k_bwd_dq_ds<DQK, VL>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       C::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((k_bwd_dq_ds<DQK, VL>), dim3(unsigned(grid)), dim3(C::NT), C::LDS_BYTES, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_split_ds_dq(const BwdArgs& a, hipStream_t s) {
    const bool vl = a.cu_q != nullptr;             // packed sequences
    switch (a.Dqk) {
        case 64: return vl ? launch_t<64, true>(a, s) : launch_t<64, false>(a, s);
        case 128: return vl ? launch_t<128, true>(a, s) : launch_t<128, false>(a, s);
        case 192: return vl ? launch_t<192, true>(a, s) : launch_t<192, false>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace isattn
