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
    const float* lse;     // [B, Hq, lse_ld] natural-log LSE
    float* delta;         // [B, Hq, stat_ld] workspace: rowsum(dO * O); SPLIT / SPLIT_DS store its negation
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
    // SPLIT_DS: bf16 dS tiles of 128 x 128, one per kept (b, h, qb, kb) block
    // (dS tile slots below); else null.  ds_cap: tiles the workspace holds
    // (fewer than 2^31), ds_T: tiles per (b, h) of a dense mask.  Block CSR
    // masks: ds_map[p] is the K->Q position of Q->K entry p (ds_map_len
    // entries; -1 where the two forms disagree), and *ds_flag is set when the
    // CSR's true block count needs more than ds_cap tiles (both passes then
    // compute nothing; reads of a tile are clamped into [0, ds_cap) anyway).
    uint16_t* ds;
    int32_t ds_cap, ds_T;
    int32_t* ds_map;
    int32_t* ds_flag;
    int64_t ds_map_len;
    float* acc0;          // LoopK: dK accumulator [B,Hk,Sk,Dqk]; LoopQ: dQ accumulator [B,Hq,Sq,Dqk]
    float* acc1;          // LoopK: dV accumulator [B,Hk,Sk,Dv]; LoopQ: unused
    int64_t acc0_elems, acc1_elems;
    // block CSR (mask_kind == 1)
    const int32_t* q2k_ptr; const int32_t* q2k_col;
    const int32_t* k2q_ptr; const int32_t* k2q_col;
    // token-exact bits per (b, mask head, qb, kb) slot of 1024 words
    // (row-major words [0, 512), key-major [512, 1024)); null: block-granular
    const uint32_t* tok;
    // packed variable-length sequences: sequence b is tokens [cu_q[b], cu_q[b+1])
    // of the query-side tensors and [cu_k[b], cu_k[b+1]) of the key side; Sq
    // and Sk hold the longest lengths (a kernel narrows them to its sequence
    // with seq_view); null for fixed-length batches
    const int32_t* cu_q; const int32_t* cu_k;
    int32_t B, Sq, Sk, Hq, Hk, G, Dqk, Dv;
    int32_t Hm, n_qb, n_kb;
    int32_t lse_ld;       // row stride of lse per (b, h): the (longest) Sq
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
    float* lse;           // [B, Hq, lse_ld] natural-log LSE (+inf for a row with no kept key)
    const int32_t* q2k_ptr; const int32_t* q2k_col;   // block CSR (mask_kind == 1)
    const uint32_t* tok;                              // token-exact bits, as in BwdArgs
    const int32_t* cu_q; const int32_t* cu_k;         // packed sequences, as in BwdArgs
    int32_t B, Sq, Sk, Hq, Hk, G, Dqk, Dv;
    int32_t Hm, n_qb, n_kb;
    int32_t lse_ld;
    int32_t mask_kind, causal;
    float scale_log2;     // softmax_scale * log2(e)
};

#if defined(__HIPCC__)
#define ISATTN_HD __host__ __device__
#else
#define ISATTN_HD
#endif

// ---- dS tile slots of SPLIT_DS ---------------------------------------------
// Block CSR mask: the slot of (b, h, qb, kb) is R * p + (h - hm * R), with p
// the position of the block in the K->Q lists, R = Hq / Hm query heads per
// mask head and hm = h * Hm / Hq: R * nnz slots in all.  Dense masks at fixed
// lengths: (b * Hq + h) * T + (visible blocks of the query blocks before qb)
// + kb, T the visible blocks of one head (bottom-right causal cut, or all
// n_qb * n_kb without it).  Packed sequences with a dense mask: every
// (qb, kb) of the longest lengths, T = n_qb * n_kb (a sequence's causal cut
// differs from that of the longest lengths).
ISATTN_HD inline int64_t floor_div(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
// key blocks visible to query block qb: rows up to min(128 qb + 127, Sq - 1)
// see keys up to that row + Sk - Sq (all n_kb without the causal term)
ISATTN_HD inline int64_t visible_kb(int64_t qb, int64_t Sq, int64_t Sk, int64_t n_kb, bool causal) {
    if (!causal) return n_kb;
    const int64_t last_row = 128 * qb + 127 < Sq - 1 ? 128 * qb + 127 : Sq - 1;
    const int64_t last_key = last_row + Sk - Sq;
    if (last_key < 0) return 0;
    const int64_t n = last_key / 128 + 1;
    return n < n_kb ? n : n_kb;
}
// sum of clamp(x, 0, N) over the integers x < y
ISATTN_HD inline int64_t clamp_prefix(int64_t y, int64_t N) {
    if (y <= 0) return 0;
    if (y <= N + 1) return y * (y - 1) / 2;
    return N * (N + 1) / 2 + (y - N - 1) * N;
}
// visible key blocks of the query blocks before qb (qb <= n_qb - 1): blocks
// qb' < n_qb - 1 are whole, so visible_kb(qb') = clamp(qb' + c0, 0, n_kb)
// with c0 = 1 + floor((127 + Sk - Sq) / 128)
ISATTN_HD inline int64_t visible_before(int64_t qb, int64_t Sq, int64_t Sk, int64_t n_kb, bool causal) {
    if (!causal) return qb * n_kb;
    const int64_t c0 = 1 + floor_div(127 + Sk - Sq, 128);
    return clamp_prefix(c0 + qb, n_kb) - clamp_prefix(c0, n_kb);
}

#if defined(__HIPCC__)
// Narrow the arguments to packed sequence b: its lengths (clamped to the
// longest, so tiles and statistics rows stay inside their allocations) and
// tensor pointers moved so that the batch-b address arithmetic of the
// kernels (base + b * stride_b + row * stride_s) lands on its first token.
__device__ __forceinline__ int seq_len(const int32_t* cu, int b, int longest) {
    const int n = cu[b + 1] - cu[b];
    return n < 0 ? 0 : (n > longest ? longest : n);
}
template <class T>
__device__ __forceinline__ void seq_shift(T*& p, int64_t first, int64_t ss, int64_t sb, int b) {
    p += first * ss - int64_t(b) * sb;
}
__device__ __forceinline__ void seq_view(BwdArgs& a, int b) {
    const int64_t q0 = a.cu_q[b], k0 = a.cu_k[b];
    a.Sq = seq_len(a.cu_q, b, a.Sq);
    a.Sk = seq_len(a.cu_k, b, a.Sk);
    seq_shift(a.q, q0, a.q_ss, a.q_sb, b);
    seq_shift(a.o, q0, a.o_ss, a.o_sb, b);
    seq_shift(a.dO, q0, a.do_ss, a.do_sb, b);
    seq_shift(a.dq, q0, a.dq_ss, a.dq_sb, b);
    seq_shift(a.k, k0, a.k_ss, a.k_sb, b);
    seq_shift(a.v, k0, a.v_ss, a.v_sb, b);
    seq_shift(a.dk, k0, a.dk_ss, a.dk_sb, b);
    seq_shift(a.dv, k0, a.dv_ss, a.dv_sb, b);
}
__device__ __forceinline__ void seq_view(FwdArgs& a, int b) {
    const int64_t q0 = a.cu_q[b], k0 = a.cu_k[b];
    a.Sq = seq_len(a.cu_q, b, a.Sq);
    a.Sk = seq_len(a.cu_k, b, a.Sk);
    seq_shift(a.q, q0, a.q_ss, a.q_sb, b);
    seq_shift(a.o, q0, a.o_ss, a.o_sb, b);
    seq_shift(a.k, k0, a.k_ss, a.k_sb, b);
    seq_shift(a.v, k0, a.v_ss, a.v_sb, b);
}
#endif

}  // namespace isattn
