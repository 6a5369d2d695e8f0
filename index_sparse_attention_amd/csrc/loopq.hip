// LoopQ attention backward: outer loop over key tiles, inner loop over the
// kept query tiles of every query head of the GQA group (the default
// direction that MagiAttention PR #334 compares LoopK against: dK/dV stay on
// chip, dQ is reduced by fp32 atomics; the key-block -> query-block lists are
// the K2Q CSR metadata of MagiAttention PR #331, "CSR Tile Mapping").  dK/dV
// are written directly as bf16 once the group is done (no postprocess for
// them, as the flash-attention "switch mha to no postprocess" commit does).
//
// One workgroup = 4 waves = one 128-key tile of one (batch, KV head); wave w
// owns keys 32w..32w+31.  Each inner step stages 64 query rows of Q and dO
// (rows swap23-staged and chunk-swizzled, so the dV / dK B operands come from
// transposing reads), their LSE*log2e and delta; the next step's rows are
// loaded into registers while the current one computes.  Per step and wave:
//
//   S  = Q K^T        [64 q x 32 keys]  32x32x16 MFMA, A = Q (LDS), B = K (regs)
//   dP = dO V^T       [64 q x 32 keys]  B = V (regs)
//   P  = exp2(S*scale*log2e - LSE*log2e),  dS = P * (dP - delta)
//   dV += P^T dO      [32 keys x Dv]    A = P^T from the S accumulator registers
//   dK += dS^T Q      [32 keys x Dqk]   A = dS^T from registers, B = Q^T (LDS,
//                                       transposing reads)
//   dS -> LDS, then dQ_part = dS K [64 q x Dqk/4] per wave (16x16x32 MFMA,
//   B = K (regs)), fp32 atomic add into the dQ accumulator.
#include "device_common.hpp"
#include "kernels.hpp"

namespace isattn {
namespace {


template <int DQK, int DV>
struct LoopQCfg {
    static constexpr int BN = 128;                 // keys per workgroup
    static constexpr int BM = 64;                  // query rows per inner step
    static constexpr int NT = 256;
    static constexpr int PDS = BN + 8;             // sdS[m][key]
    // Q and dO tiles: rows swap23-staged, 16-byte chunks swizzled, no padding
    // (the layout the transposing operand reads expect)
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_DO = OFF_Q + BM * DQK;
    static constexpr int OFF_DS = OFF_DO + BM * DV;
    static constexpr int OFF_STAT = OFF_DS + BM * PDS;  // float lse2[BM], delta[BM]
    static constexpr int END_LOOP = OFF_STAT + 4 * BM;
    static constexpr int PK = DQK + 8;             // prologue staging
    static constexpr int PV = DV + 8;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_V = BN * PK;
    static constexpr int END_PRO = OFF_V + BN * PV;
    static constexpr int LDS_ELEMS = END_LOOP > END_PRO ? END_LOOP : END_PRO;
    static constexpr int LDS_BYTES = LDS_ELEMS * 2;
    static constexpr int NCQ = DQK / 16;
    static constexpr int NCV = DV / 16;
    static constexpr int NDK = DQK / 32;           // dK accumulator tiles
    static constexpr int NDV = DV / 32;            // dV accumulator tiles
    static constexpr int WQ = DQK / 4;             // dQ d-slice per wave
    static constexpr int NTQ = WQ / 16;
    static_assert(WQ % 16 == 0, "Dqk must split into 16-wide tiles per wave");
    static_assert((OFF_STAT * 2) % 16 == 0, "stat block alignment");
};

template <int D, int PITCH, int ROWS, int NT>
__device__ __forceinline__ void stage_rows(uint16_t* dst, const uint16_t* src, int64_t row_stride,
                                           int row0, int limit, int tid) {
    TileStager<D, PITCH, ROWS, NT, false> t;
    t.load(src, row_stride, row0, limit, tid);
    t.store(dst, tid);
}

// ROWS rows: row-major copy (pitch P) and transposed copy (pitch PT).
template <int D, int P, int PT, int ROWS, int NT>
__device__ __forceinline__ void stage_both(uint16_t* dst, uint16_t* dstT, const uint16_t* src,
                                           int64_t row_stride, int row0, int limit, int tid) {
    TileStager<D, P, ROWS, NT, false> t;
    t.load(src, row_stride, row0, limit, tid);
    t.store(dst, tid);
    t.template store_t<PT>(dstT, tid);
}

template <int DQK, int DV>
__global__ __launch_bounds__(256, 1) void k_bwd_loopq(BwdArgs a) {
    using C = LoopQCfg<DQK, DV>;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31, h2 = lane >> 5;
    const int l16 = lane & 15, g4 = lane >> 4;

    // ---- work item: longest key columns first under a causal mask
    const int BH = a.B * a.Hk;
    const int id = blockIdx.x;
    const int kb = id / BH;
    const int bh = id - kb * BH;
    const int b = bh / a.Hk;
    const int hk = bh - b * a.Hk;
    const int n_base = kb * C::BN;
    const int shift = a.Sk - a.Sq;

    // ---- prologue: K and V tiles -> registers
    stage_rows<DQK, C::PK, C::BN, C::NT>(lds + C::OFF_K, a.k + b * a.k_sb + hk * a.k_sh, a.k_ss, n_base,
                                         a.Sk, tid);
    stage_rows<DV, C::PV, C::BN, C::NT>(lds + C::OFF_V, a.v + b * a.v_sb + hk * a.v_sh, a.v_ss, n_base,
                                        a.Sk, tid);
    __syncthreads();
    const int nk = 32 * w + l32;                 // this lane's key within the tile (32x32 column)
    bf16x8_t kS[C::NCQ], vS[C::NCV];             // B operands of S / dP
    bf16x8_t kQ[C::NTQ][4];                      // B operand of dQ_part (k = key)
    {
        const uint16_t* sK = lds + C::OFF_K;
        const uint16_t* sV = lds + C::OFF_V;
#pragma unroll
        for (int c = 0; c < C::NCQ; ++c) kS[c] = as_bf16x8(lds_read128(sK + nk * C::PK + 16 * c + 8 * h2));
#pragma unroll
        for (int c = 0; c < C::NCV; ++c) vS[c] = as_bf16x8(lds_read128(sV + nk * C::PV + 16 * c + 8 * h2));
#pragma unroll
        for (int t = 0; t < C::NTQ; ++t) {
            const int d = w * C::WQ + 16 * t + l16;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u32x4_t v;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = 32 * c + 8 * g4 + 2 * j;
                    v[j] = uint32_t(sK[n * C::PK + d]) | (uint32_t(sK[(n + 1) * C::PK + d]) << 16);
                }
                kQ[t][c] = as_bf16x8(v);
            }
        }
    }
    __syncthreads();

    f32x16_t dk[C::NDK], dv[C::NDV];
#pragma unroll
    for (int t = 0; t < C::NDK; ++t) dk[t] = f32x16_t{};
#pragma unroll
    for (int t = 0; t < C::NDV; ++t) dv[t] = f32x16_t{};

    uint16_t* sQ = lds + C::OFF_Q;
    uint16_t* sdO = lds + C::OFF_DO;
    uint16_t* sdS = lds + C::OFF_DS;
    float* sL = reinterpret_cast<float*>(lds + C::OFF_STAT);
    float* sD = sL + C::BM;
    const int key = n_base + nk;
    const bool key_in = key < a.Sk;
    const bool tile_ragged = n_base + C::BN > a.Sk;

    // ---- steps: every 64-row half of every kept query block (of every query
    // head of the GQA group) that some row of sees the key tile, in order.
    // The next step's Q and dO rows and statistics are loaded into registers
    // while the current step computes and issues its dQ atomics, and staged
    // into LDS once the step is done.
    struct Step {
        int gi, it, half, m0;
    };
    int cnt = 0, first = 0, chunk = -1, chunk_base = -1;
    const int32_t* list = nullptr;
    auto head_list = [&](int gi) {
        const int h = hk * a.G + gi;
        list = nullptr;
        first = 0;
        chunk_base = -1;
        if (a.mask_kind == 1) {
            const int hm = h * a.Hm / a.Hq;
            const int r = (b * a.Hm + hm) * a.n_kb + kb;
            const int beg = a.k2q_ptr[r];
            cnt = a.k2q_ptr[r + 1] - beg;
            list = a.k2q_col + beg;
        } else {
            if (a.causal) {
                const int first_row = n_base - shift;           // first row that sees key n_base
                first = first_row <= 0 ? 0 : first_row / kBlock;
            }
            cnt = a.n_qb - first;
        }
    };
    auto qb_at = [&](int it) {
        if (list == nullptr) return first + it;
        const int base = it & ~63;
        if (base != chunk_base) {
            chunk_base = base;
            chunk = base + lane < cnt ? list[base + lane] : -1;
        }
        return __builtin_amdgcn_readlane(chunk, it & 63);
    };
    // the step after st (st.gi < 0: before the first); gi == G: none left
    constexpr int PARTS = kBlock / C::BM;
    auto advance = [&](Step st) {
        if (st.gi < 0) {
            st.gi = 0;
            head_list(0);
            st.it = 0;
            st.half = -1;
        }
        for (;;) {
            if (++st.half >= PARTS) {
                st.half = 0;
                ++st.it;
            }
            while (st.it >= cnt) {                  // the head's list is done
                if (++st.gi >= a.G) return st;
                head_list(st.gi);
                st.it = 0;
                st.half = 0;
            }
            const int qb = qb_at(st.it);
            if (qb < 0 || qb >= a.n_qb) {           // ignore malformed CSR entries
                st.half = PARTS - 1;
                continue;
            }
            st.m0 = qb * kBlock + st.half * C::BM;
            if (st.m0 >= a.Sq) {                    // the block's remaining rows are past Sq
                st.half = PARTS - 1;
                continue;
            }
            const int mlast = min(st.m0 + C::BM - 1, a.Sq - 1);
            if (a.causal && mlast + shift < n_base) continue;  // every row of the step precedes the tile
            return st;
        }
    };
    TileStager<DQK, DQK, C::BM, C::NT, true> tq;
    TileStager<DV, DV, C::BM, C::NT, true> tdo;
    // raw statistics of the next step's row tid; scaled and masked when staged,
    // so nothing waits on these loads before the step's work is issued
    float nl = 0.f, nd = 0.f;
    bool nin = false;
    auto issue = [&](const Step& st) {              // loads of step st into registers
        const int h = hk * a.G + st.gi;
        tq.load(a.q + b * a.q_sb + h * a.q_sh, a.q_ss, st.m0, a.Sq, tid);
        tdo.load(a.dO + b * a.do_sb + h * a.do_sh, a.do_ss, st.m0, a.Sq, tid);
        if (tid < C::BM) {
            const int64_t srow = (int64_t(b) * a.Hq + h) * a.Sq;
            const int row = st.m0 + tid;
            nin = row < a.Sq;
            if (nin) {
                nl = a.lse[srow + row];
                nd = a.delta[srow + row];
            }
        }
    };

    Step cur = advance(Step{-1, 0, 0, 0});
    if (cur.gi < a.G) issue(cur);
    while (cur.gi < a.G) {
        const int m0 = cur.m0;
        const int h = hk * a.G + cur.gi;
        float* gdq = a.acc0 + (int64_t(b) * a.Hq + h) * a.Sq * DQK;   // head-major [B, Hq, Sq, Dqk]
        tq.store_swz(sQ, tid);
        tdo.store_swz(sdO, tid);
        if (tid < C::BM) {
            sL[tid] = nin ? nl * kLog2e : __builtin_inff();
            sD[tid] = nin ? nd : 0.f;
        }
        __syncthreads();
        const Step nxt = advance(cur);
        if (nxt.gi < a.G) issue(nxt);
        {
                f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
                f32x16_t dp[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
                for (int c = 0; c < C::NCQ; ++c) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const bf16x8_t qa = as_bf16x8(lds_read128(sQ + 32 * mt * DQK + swz_off<DQK>(l32, 16 * c + 8 * h2)));
                        s[mt] = mfma32(qa, kS[c], s[mt]);
                    }
                }
#pragma unroll
                for (int c = 0; c < C::NCV; ++c) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const bf16x8_t oa = as_bf16x8(lds_read128(sdO + 32 * mt * DV + swz_off<DV>(l32, 16 * c + 8 * h2)));
                        dp[mt] = mfma32(oa, vS[c], dp[mt]);
                    }
                }

                const bool need_mask = tile_ragged || (a.causal && n_base + C::BN - 1 > m0 + shift);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        // LDS row 32 mt + 8 (i / 4) + 4 h2 + i % 4 holds logical row swap23 of it
                        const int ml = 32 * mt + swap23(8 * (i >> 2) + 4 * h2 + (i & 3));
                        float p = fast_exp2(s[mt][i] * a.scale_log2 - sL[ml]);
                        if (need_mask) {
                            const bool ok = key_in && (!a.causal || key <= m0 + ml + shift);
                            p = ok ? p : 0.f;
                        }
                        const float ds = p * (dp[mt][i] - sD[ml]);
                        s[mt][i] = p;
                        dp[mt][i] = ds;
                        sdS[ml * C::PDS + nk] = to_bf16(ds);
                    }
                }

                // dV += P^T dO, dK += dS^T Q  (A operands straight from registers)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        u32x4_t pp, pd;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            pp[j] = pack_bf16x2(s[mt][8 * c + 2 * j], s[mt][8 * c + 2 * j + 1]);
                            pd[j] = pack_bf16x2(dp[mt][8 * c + 2 * j], dp[mt][8 * c + 2 * j + 1]);
                        }
                        // k = logical rows 32 mt + 16 c + 8 h2 + 0..7: the partner
                        // columns by transposing reads of the swizzled tiles
                        const int roff = 32 * mt + 16 * c;
#pragma unroll
                        for (int dt = 0; dt < C::NDV; ++dt) {
                            const u32x2_t lo = lds_read_tr16(sdO + roff * DV + tr_read_off<DV>(lane, dt, 0) / 2);
                            const u32x2_t hi = lds_read_tr16(sdO + roff * DV + tr_read_off<DV>(lane, dt, 1) / 2);
                            const u32x4_t bv = {lo[0], lo[1], hi[0], hi[1]};
                            dv[dt] = mfma32(as_bf16x8(pp), as_bf16x8(bv), dv[dt]);
                        }
#pragma unroll
                        for (int dt = 0; dt < C::NDK; ++dt) {
                            const u32x2_t lo = lds_read_tr16(sQ + roff * DQK + tr_read_off<DQK>(lane, dt, 0) / 2);
                            const u32x2_t hi = lds_read_tr16(sQ + roff * DQK + tr_read_off<DQK>(lane, dt, 1) / 2);
                            const u32x4_t bq = {lo[0], lo[1], hi[0], hi[1]};
                            dk[dt] = mfma32(as_bf16x8(pd), as_bf16x8(bq), dk[dt]);
                        }
                    }
                }
                __syncthreads();

                // dQ_part = dS K on this wave's d-slice; atomics into the dQ accumulator
#pragma unroll
                for (int mt = 0; mt < C::BM / 16; ++mt) {
                    bf16x8_t sa[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        sa[c] = as_bf16x8(lds_read128(sdS + (16 * mt + l16) * C::PDS + 32 * c + 8 * g4));
                    const int row0 = m0 + 16 * mt + 4 * g4;
#pragma unroll
                    for (int t = 0; t < C::NTQ; ++t) {
                        f32x4_t acc = f32x4_t{};
#pragma unroll
                        for (int c = 0; c < 4; ++c) acc = mfma16(sa[c], kQ[t][c], acc);
                        const int d = w * C::WQ + 16 * t + l16;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (row0 + i < a.Sq)
                                atomic_add_f32(gdq + int64_t(row0 + i) * DQK + d, acc[i]);
                    }
                }
                __syncthreads();
        }
        cur = nxt;
    }

    // ---- epilogue: dK = scale * acc, dV = acc -> bf16, stored directly
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

template <int DQK, int DV>
hipError_t launch_t(const BwdArgs& a, hipStream_t s) {
    using C = LoopQCfg<DQK, DV>;
    const int64_t grid = int64_t(a.n_kb) * a.B * a.Hk;
    if (grid == 0) return hipSuccess;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k_bwd_loopq<DQK, DV>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       C::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((k_bwd_loopq<DQK, DV>), dim3(unsigned(grid)), dim3(C::NT), C::LDS_BYTES, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_loopq(const BwdArgs& a, hipStream_t s) {
    if (a.Dqk == 64 && a.Dv == 64) return launch_t<64, 64>(a, s);
    if (a.Dqk == 128 && a.Dv == 128) return launch_t<128, 128>(a, s);
    if (a.Dqk == 192 && a.Dv == 128) return launch_t<192, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace isattn
