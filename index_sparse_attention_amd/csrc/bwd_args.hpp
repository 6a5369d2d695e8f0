// Launch arguments shared by the host dispatcher and the attention-backward
// kernels.  Plain data only: device pointers, element strides and sizes.
#pragma once
#include <stdint.h>

namespace isattn {

constexpr int kBlock = 128;   // mask block (query rows x keys) of the block-sparse path
// SPLIT dK/dV pass with fewer (b, KV head, key block) items than twice the
// CUs of an MI355X: items are cut into parts over their query-block lists
// (the "part mode"), parts of one item write fp32 partial dK/dV that a
// reduction sums in part order.
constexpr int kPartModeItems = 512;
constexpr int kMaxParts = 64;

struct BwdArgs {
    // bf16 tensors [batch, seq, heads, dim], last dim contiguous, strides in elements
    const uint16_t* q;  int64_t q_sb, q_ss, q_sh;
    const uint16_t* k;  int64_t k_sb, k_ss, k_sh;
    const uint16_t* v;  int64_t v_sb, v_ss, v_sh;
    const uint16_t* o;  int64_t o_sb, o_ss, o_sh;
    const uint16_t* dO; int64_t do_sb, do_ss, do_sh;
    uint16_t* dq; int64_t dq_sb, dq_ss, dq_sh;
    uint16_t* dk; int64_t dk_sb, dk_ss, dk_sh;
    uint16_t* dv; int64_t dv_sb, dv_ss, dv_sh;
    const float* lse;     // [B, Hq, Sq] natural-log LSE
    float* delta;         // [B, Hq, stat_ld] workspace: rowsum(dO * O)
    float* lse2;          // [B, Hq, stat_ld] workspace (SPLIT only): lse * log2(e); else null
    int32_t* order;       // SPLIT work order: B*Hk*n_kb dK/dV items, then B*Hq*n_qb dQ items; else null
    // SPLIT part mode (kv_parts_T > 0): target blocks per part, the units
    // (item << 6 | part) in longest-first order with their count in units[bound],
    // per item {work, parts, partial slot}, and the fp32 partial dK|dV slots
    // [slot][128 keys][Dqk + Dv]
    int32_t kv_parts_T, kv_units_bound;
    int32_t* units;
    int32_t* item_info;
    float* partial;
    uint16_t* ds;         // SPLIT_DS: bf16 dS tiles [B, Hq, n_qb, n_kb][128 x 128]; else null
    float* acc0;          // LoopK: dK accumulator [B,Hk,Sk,Dqk]; LoopQ: dQ accumulator [B,Hq,Sq,Dqk]
    float* acc1;          // LoopK: dV accumulator [B,Hk,Sk,Dv]; LoopQ: unused
    int64_t acc0_elems, acc1_elems;
    // block CSR (mask_kind == 1)
    const int32_t* q2k_ptr; const int32_t* q2k_col;
    const int32_t* k2q_ptr; const int32_t* k2q_col;
    int32_t B, Sq, Sk, Hq, Hk, G, Dqk, Dv;
    int32_t Hm, n_qb, n_kb;
    int32_t stat_ld;      // row stride of delta / lse2 per (b, h): Sq, or n_qb * 128 for SPLIT
                          // (rows Sq.. hold delta = 0, lse2 = +inf)
    int32_t mask_kind, causal;
    float scale;          // softmax_scale
    float scale_log2;     // softmax_scale * log2(e)
};

// Launch arguments of the forward (O and LSE from Q, K, V and the mask).
struct FwdArgs {
    const uint16_t* q; int64_t q_sb, q_ss, q_sh;
    const uint16_t* k; int64_t k_sb, k_ss, k_sh;
    const uint16_t* v; int64_t v_sb, v_ss, v_sh;
    uint16_t* o; int64_t o_sb, o_ss, o_sh;
    float* lse;           // [B, Hq, Sq] natural-log LSE (+inf for a row with no kept key)
    const int32_t* q2k_ptr; const int32_t* q2k_col;   // block CSR (mask_kind == 1)
    int32_t B, Sq, Sk, Hq, Hk, G, Dqk, Dv;
    int32_t Hm, n_qb, n_kb;
    int32_t mask_kind, causal;
    float scale_log2;     // softmax_scale * log2(e)
};

}  // namespace isattn
