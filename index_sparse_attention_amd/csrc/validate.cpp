// Host-side argument checking and workspace planning (no HIP calls).
#include "validate.hpp"

#include <algorithm>

#include <cmath>
#include <limits>

namespace isattn {

namespace {

bool supported_dims(int32_t dqk, int32_t dv) {
    return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A bf16 [b, s, h, d] view: pointer present when it has elements, 16-byte
// aligned rows, non-negative strides in multiples of 8 elements.
isattn_status_t check_view(const isattn_tensor_t* t, int64_t elems) {
    if (t == nullptr) return ISATTN_ERR_NULL;
    if (elems == 0) return ISATTN_OK;
    if (t->ptr == nullptr) return ISATTN_ERR_NULL;
    if (!aligned16(t->ptr)) return ISATTN_ERR_STRIDE_ALIGN;
    if (t->stride_b < 0 || t->stride_s < 0 || t->stride_h < 0) return ISATTN_ERR_STRIDE_ALIGN;
    if ((t->stride_b % 8) || (t->stride_s % 8) || (t->stride_h % 8)) return ISATTN_ERR_STRIDE_ALIGN;
    return ISATTN_OK;
}

void copy_view(const isattn_tensor_t* t, const uint16_t** p, int64_t* sb, int64_t* ss, int64_t* sh) {
    *p = static_cast<const uint16_t*>(t->ptr);
    *sb = t->stride_b;
    *ss = t->stride_s;
    *sh = t->stride_h;
}

void copy_view_out(const isattn_tensor_t* t, uint16_t** p, int64_t* sb, int64_t* ss, int64_t* sh) {
    *p = static_cast<uint16_t*>(t->ptr);
    *sb = t->stride_b;
    *ss = t->stride_s;
    *sh = t->stride_h;
}

}  // namespace

bool plan_bwd_workspace(const isattn_shape_t& s, int32_t algo, BwdPlan* plan, const MaskInfo& mask,
                        bool allow_parts) {
    if (s.batch < 0 || s.seqlen_q < 0 || s.seqlen_k < 0 || s.heads_q < 1 || s.heads_k < 1)
        return false;
    if (algo != ISATTN_ALGO_LOOPK && algo != ISATTN_ALGO_LOOPQ && algo != ISATTN_ALGO_SPLIT &&
        algo != ISATTN_ALGO_SPLIT_DS)
        return false;
    const bool split = algo == ISATTN_ALGO_SPLIT || algo == ISATTN_ALGO_SPLIT_DS;
    BwdPlan p{};
    p.n_qb = cdiv(s.seqlen_q, kBlock);
    p.n_kb = cdiv(s.seqlen_k, kBlock);
    p.G = s.heads_k > 0 ? s.heads_q / s.heads_k : 0;
    const int64_t rows_q = int64_t(s.batch) * s.seqlen_q * s.heads_q;
    const int64_t rows_k = int64_t(s.batch) * s.seqlen_k * s.heads_k;
    // SPLIT and SPLIT_DS pad the per-row statistics of each (b, h) to whole 128-row blocks
    p.stat_ld = split ? p.n_qb * kBlock : s.seqlen_q;
    const int64_t stat_rows = int64_t(s.batch) * s.heads_q * p.stat_ld;
    size_t off = 0;
    p.off_delta = off;
    off = align_up(off + size_t(stat_rows) * sizeof(float), kWsAlign);
    p.off_lse2 = off;
    if (split) off = align_up(off + size_t(stat_rows) * sizeof(float), kWsAlign);
    // SPLIT: work order of the two passes (dK/dV items, then dQ items)
    p.off_order = off;
    if (split) {
        const int64_t items = int64_t(s.batch) * (int64_t(s.heads_k) * p.n_kb + int64_t(s.heads_q) * p.n_qb);
        off = align_up(off + size_t(items) * sizeof(int32_t), kWsAlign);
    }
    // SPLIT part mode: few dK/dV items, each cut into parts of about T
    // query blocks.  A part costs a fixed amount (its pipeline start and
    // drain, its fp32 partial written and reduced) and the last parts leave
    // CUs idle for about T / 2 blocks, so T grows with the square root of
    // the work per CU (dense-equivalent work over the 256 CUs)
    p.kv_parts_T = 0;
    p.kv_units_bound = 0;
    p.off_units = p.off_info = p.off_partial = off;
    const int64_t n_kv = int64_t(s.batch) * s.heads_k * p.n_kb;
    if (split && allow_parts && n_kv > 0 && n_kv < kPartModeItems) {
        const int64_t per_item = int64_t(p.G) * p.n_qb;      // query blocks of an item, dense
        const int64_t T = std::max<int64_t>(1, int64_t(std::ceil(std::sqrt(16.0 * double(per_item * n_kv) / 256.0))));
        const int64_t pmax = std::min<int64_t>(kMaxParts, std::max<int64_t>(1, (per_item + T - 1) / T));
        p.kv_parts_T = int32_t(T);
        p.kv_units_bound = int32_t(n_kv * pmax);
        p.off_units = off;
        off = align_up(off + size_t(p.kv_units_bound + 1) * sizeof(int32_t), kWsAlign);
        p.off_info = off;
        off = align_up(off + size_t(3 * n_kv) * sizeof(int32_t), kWsAlign);
        p.off_partial = off;
        off = align_up(off + size_t(p.kv_units_bound) * kBlock * (s.dim_qk + s.dim_v) * sizeof(float), kWsAlign);
    }
    if (algo == ISATTN_ALGO_LOOPK) {
        p.acc0_elems = rows_k * s.dim_qk;
        p.acc1_elems = rows_k * s.dim_v;
    } else if (algo == ISATTN_ALGO_LOOPQ) {
        p.acc0_elems = rows_q * s.dim_qk;
        p.acc1_elems = 0;
    } else {
        p.acc0_elems = 0;
        p.acc1_elems = 0;
    }
    p.off_acc0 = off;
    off = align_up(off + size_t(p.acc0_elems) * sizeof(float), kWsAlign);
    p.off_acc1 = off;
    off = align_up(off + size_t(p.acc1_elems) * sizeof(float), kWsAlign);
    // SPLIT_DS: for a block CSR the K->Q position of every Q->K entry, then a
    // bf16 dS tile for every kept block of every query head (the slots of
    // ds_slot in bwd_args.hpp)
    p.ds_tiles = p.ds_T = p.ds_map_len = 0;
    if (algo == ISATTN_ALGO_SPLIT_DS) {
        const int64_t grid = int64_t(p.n_qb) * p.n_kb;
        const int64_t bh = int64_t(s.batch) * s.heads_q;
        if (mask.kind == ISATTN_MASK_BLOCK_CSR) {
            const int64_t hm = mask.heads > 0 ? mask.heads : s.heads_q;
            p.ds_map_len = mask.nnz >= 0 ? mask.nnz : int64_t(s.batch) * hm * grid;
            p.ds_tiles = (s.heads_q / hm) * p.ds_map_len;
        } else if (mask.kind == ISATTN_MASK_DENSE) {
            p.ds_T = mask.varlen ? grid
                                 : visible_before(p.n_qb - 1, s.seqlen_q, s.seqlen_k, p.n_kb, mask.causal) +
                                       visible_kb(p.n_qb - 1, s.seqlen_q, s.seqlen_k, p.n_kb, mask.causal);
            if (p.n_qb == 0) p.ds_T = 0;
            p.ds_tiles = bh * p.ds_T;
        } else {                                     // mask unknown: every block, a map for Hq mask heads
            p.ds_map_len = bh * grid;
            p.ds_tiles = bh * grid;
        }
    }
    // the position map and, after it, the int32 overflow flag of a block CSR
    p.off_dsmap = off;
    if (algo == ISATTN_ALGO_SPLIT_DS && mask.kind != ISATTN_MASK_DENSE)
        off = align_up(off + size_t(p.ds_map_len + 1) * sizeof(int32_t), kWsAlign);
    p.off_ds = off;
    off = align_up(off + size_t(p.ds_tiles) * kBlock * kBlock * 2, kWsAlign);
    p.total = off;
    *plan = p;
    return true;
}

isattn_status_t validate_bwd(const isattn_shape_t* shape, const isattn_tensor_t* q,
                             const isattn_tensor_t* k, const isattn_tensor_t* v,
                             const isattn_tensor_t* o, const isattn_tensor_t* dO,
                             const float* lse, const isattn_mask_t* mask, int32_t causal,
                             float softmax_scale, const isattn_tensor_t* dq,
                             const isattn_tensor_t* dk, const isattn_tensor_t* dv, int32_t algo,
                             const void* workspace, size_t workspace_bytes, BwdArgs* args,
                             BwdPlan* plan, const isattn_varlen_t* varlen, bool allow_parts) {
    if (shape == nullptr) return ISATTN_ERR_NULL;
    const isattn_shape_t s = *shape;
    if (s.batch < 0 || s.seqlen_q < 0 || s.seqlen_k < 0 || s.heads_q < 1 || s.heads_k < 1)
        return ISATTN_ERR_SHAPE;
    if (s.heads_q % s.heads_k != 0) return ISATTN_ERR_SHAPE;
    if (s.seqlen_q >= (1 << 30) || s.seqlen_k >= (1 << 30)) return ISATTN_ERR_SHAPE;
    // block-level work items (padded to a multiple of 8 workgroups) must fit an int
    if (int64_t(s.batch) * s.heads_q * cdiv(s.seqlen_q, kBlock) >= (int64_t(1) << 31) - 8 ||
        int64_t(s.batch) * s.heads_k * cdiv(s.seqlen_k, kBlock) >= (int64_t(1) << 31) - 8)
        return ISATTN_ERR_SHAPE;
    if (!supported_dims(s.dim_qk, s.dim_v)) return ISATTN_ERR_UNSUPPORTED;
    if (algo != ISATTN_ALGO_LOOPK && algo != ISATTN_ALGO_LOOPQ && algo != ISATTN_ALGO_SPLIT &&
        algo != ISATTN_ALGO_SPLIT_DS)
        return ISATTN_ERR_UNSUPPORTED;
    if (!std::isfinite(softmax_scale)) return ISATTN_ERR_UNSUPPORTED;

    const int64_t nq = int64_t(s.batch) * s.seqlen_q * s.heads_q;
    const int64_t nk = int64_t(s.batch) * s.seqlen_k * s.heads_k;
    isattn_status_t st;
    if ((st = check_view(q, nq)) != ISATTN_OK) return st;
    if ((st = check_view(k, nk)) != ISATTN_OK) return st;
    if ((st = check_view(v, nk)) != ISATTN_OK) return st;
    if ((st = check_view(o, nq)) != ISATTN_OK) return st;
    if ((st = check_view(dO, nq)) != ISATTN_OK) return st;
    if ((st = check_view(dq, nq)) != ISATTN_OK) return st;
    if ((st = check_view(dk, nk)) != ISATTN_OK) return st;
    if ((st = check_view(dv, nk)) != ISATTN_OK) return st;
    if (nq > 0 && lse == nullptr) return ISATTN_ERR_NULL;
    if ((algo == ISATTN_ALGO_SPLIT || algo == ISATTN_ALGO_SPLIT_DS) && nq > 0) {
        // 32-bit byte offsets within one head: Q/dO rows (dK/dV pass), K/V rows (dQ pass)
        const int64_t lim = int64_t(1) << 31;
        const int64_t rq = int64_t(cdiv(s.seqlen_q, kBlock)) * kBlock;
        const int64_t rk = int64_t(cdiv(s.seqlen_k, kBlock)) * kBlock;
        if (rq * q->stride_s * 2 >= lim || rq * dO->stride_s * 2 >= lim || rk * k->stride_s * 2 >= lim ||
            rk * v->stride_s * 2 >= lim)
            return ISATTN_ERR_STRIDE_ALIGN;
    }

    BwdArgs a{};
    a.mask_kind = ISATTN_MASK_DENSE;
    a.Hm = 0;
    if (mask != nullptr && mask->kind != ISATTN_MASK_DENSE) {
        if (mask->kind != ISATTN_MASK_BLOCK_CSR) return ISATTN_ERR_MASK;
        if (mask->block_q != kBlock || mask->block_k != kBlock) return ISATTN_ERR_UNSUPPORTED;
        if (mask->heads != 1 && mask->heads != s.heads_k && mask->heads != s.heads_q)
            return ISATTN_ERR_MASK;
        if (algo != ISATTN_ALGO_LOOPQ && (mask->q2k_row_ptr == nullptr || mask->q2k_col == nullptr))
            return ISATTN_ERR_NULL;
        if (algo != ISATTN_ALGO_LOOPK && (mask->k2q_row_ptr == nullptr || mask->k2q_col == nullptr))
            return ISATTN_ERR_NULL;
        a.mask_kind = ISATTN_MASK_BLOCK_CSR;
        a.Hm = mask->heads;
        a.q2k_ptr = mask->q2k_row_ptr;
        a.q2k_col = mask->q2k_col;
        a.k2q_ptr = mask->k2q_row_ptr;
        a.k2q_col = mask->k2q_col;
        if (mask->token_bits != nullptr) {
            // token-exact masks: the two-pass algorithms only
            if (algo != ISATTN_ALGO_SPLIT && algo != ISATTN_ALGO_SPLIT_DS) return ISATTN_ERR_UNSUPPORTED;
            if ((reinterpret_cast<uintptr_t>(mask->token_bits) & 15u) != 0) return ISATTN_ERR_STRIDE_ALIGN;
            a.tok = mask->token_bits;
        }
    }

    if (varlen != nullptr) {
        // packed sequences: the two-pass algorithms only (LoopK is fixed-length
        // only, [P1] Limitations; LoopQ follows it)
        if (algo != ISATTN_ALGO_SPLIT && algo != ISATTN_ALGO_SPLIT_DS) return ISATTN_ERR_UNSUPPORTED;
        if (s.batch > 0 && (varlen->cu_seqlens_q == nullptr || varlen->cu_seqlens_k == nullptr))
            return ISATTN_ERR_NULL;
        a.cu_q = varlen->cu_seqlens_q;
        a.cu_k = varlen->cu_seqlens_k;
    }

    MaskInfo mi;
    mi.kind = a.mask_kind;
    mi.heads = a.Hm;
    mi.nnz = a.mask_kind == ISATTN_MASK_BLOCK_CSR ? mask->nnz : -1;
    mi.causal = causal != 0;
    mi.varlen = varlen != nullptr;
    BwdPlan p{};
    if (!plan_bwd_workspace(s, algo, &p, mi, allow_parts)) return ISATTN_ERR_SHAPE;
    if (algo == ISATTN_ALGO_SPLIT_DS) {
        // the dS tiles: what the workspace holds past the fixed part, at
        // least what the mask needs
        if (workspace_bytes < p.off_ds) return ISATTN_ERR_WORKSPACE;
        const int64_t cap = int64_t((workspace_bytes - p.off_ds) / (size_t(kBlock) * kBlock * 2));
        if (cap < p.ds_tiles) return ISATTN_ERR_CAPACITY;
        if (p.ds_tiles >= INT32_MAX) return ISATTN_ERR_UNSUPPORTED;   // tile slots are int32
        a.ds_cap = int32_t(std::min<int64_t>(cap, INT32_MAX));
    } else if (workspace_bytes < p.total) {
        return ISATTN_ERR_WORKSPACE;
    }
    if (p.total > 0 && workspace == nullptr) return ISATTN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kWsAlign - 1)) != 0) return ISATTN_ERR_WORKSPACE;

    copy_view(q, &a.q, &a.q_sb, &a.q_ss, &a.q_sh);
    copy_view(k, &a.k, &a.k_sb, &a.k_ss, &a.k_sh);
    copy_view(v, &a.v, &a.v_sb, &a.v_ss, &a.v_sh);
    copy_view(o, &a.o, &a.o_sb, &a.o_ss, &a.o_sh);
    copy_view(dO, &a.dO, &a.do_sb, &a.do_ss, &a.do_sh);
    copy_view_out(dq, &a.dq, &a.dq_sb, &a.dq_ss, &a.dq_sh);
    copy_view_out(dk, &a.dk, &a.dk_sb, &a.dk_ss, &a.dk_sh);
    copy_view_out(dv, &a.dv, &a.dv_sb, &a.dv_ss, &a.dv_sh);
    a.lse = lse;
    a.B = s.batch;
    a.Sq = s.seqlen_q;
    a.Sk = s.seqlen_k;
    a.Hq = s.heads_q;
    a.Hk = s.heads_k;
    a.G = s.heads_q / s.heads_k;
    a.Dqk = s.dim_qk;
    a.Dv = s.dim_v;
    a.n_qb = p.n_qb;
    a.n_kb = p.n_kb;
    a.lse_ld = s.seqlen_q;
    a.stat_ld = p.stat_ld;
    a.causal = causal != 0;
    a.scale = softmax_scale;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.acc0_elems = p.acc0_elems;
    a.acc1_elems = p.acc1_elems;
    a.ds_T = int32_t(p.ds_T);
    a.ds_map_len = p.ds_map_len;
    *args = a;
    *plan = p;
    return ISATTN_OK;
}

bool plan_csr_workspace(int64_t batch, int64_t heads, int64_t n_qb, int64_t n_kb,
                        bool with_presence, CsrPlan* plan) {
    if (batch < 0 || heads < 0 || n_qb < 0 || n_kb < 0) return false;
    const int64_t rq = batch * heads * n_qb;
    const int64_t rk = batch * heads * n_kb;
    if (rq >= (int64_t(1) << 31) || rk >= (int64_t(1) << 31)) return false;
    CsrPlan p{};
    p.rows_q = int32_t(rq);
    p.rows_k = int32_t(rk);
    size_t off = 0;
    p.off_presence = off;
    if (with_presence) off = align_up(off + size_t(rq) * size_t(n_kb), kWsAlign);
    p.off_qcnt = off;
    off = align_up(off + size_t(rq) * sizeof(int32_t), kWsAlign);
    p.off_kcnt = off;
    off = align_up(off + size_t(rk) * sizeof(int32_t), kWsAlign);
    p.total = off;
    *plan = p;
    return true;
}

static isattn_status_t check_csr_outputs(int64_t rows_q_total, int64_t nnz_max,
                                         const int32_t* q2k_row_ptr, const int32_t* q2k_col,
                                         const int32_t* k2q_row_ptr, const int32_t* k2q_col,
                                         int64_t col_capacity) {
    (void)rows_q_total;
    if (q2k_row_ptr == nullptr || k2q_row_ptr == nullptr) return ISATTN_ERR_NULL;
    if (nnz_max > 0 && (q2k_col == nullptr || k2q_col == nullptr)) return ISATTN_ERR_NULL;
    if (col_capacity < nnz_max) return ISATTN_ERR_CAPACITY;
    return ISATTN_OK;
}

isattn_status_t validate_fwd(const isattn_shape_t* shape, const isattn_tensor_t* q,
                             const isattn_tensor_t* k, const isattn_tensor_t* v,
                             const isattn_mask_t* mask, int32_t causal, float softmax_scale,
                             const isattn_tensor_t* o, const float* lse, FwdArgs* args,
                             const isattn_varlen_t* varlen) {
    if (shape == nullptr) return ISATTN_ERR_NULL;
    const isattn_shape_t s = *shape;
    if (s.batch < 0 || s.seqlen_q < 0 || s.seqlen_k < 0 || s.heads_q < 1 || s.heads_k < 1)
        return ISATTN_ERR_SHAPE;
    if (s.heads_q % s.heads_k != 0) return ISATTN_ERR_SHAPE;
    if (s.seqlen_q >= (1 << 30) || s.seqlen_k >= (1 << 30)) return ISATTN_ERR_SHAPE;
    if (int64_t(s.batch) * s.heads_q * cdiv(s.seqlen_q, kBlock) >= (int64_t(1) << 31) - 8)
        return ISATTN_ERR_SHAPE;
    if (!supported_dims(s.dim_qk, s.dim_v)) return ISATTN_ERR_UNSUPPORTED;
    if (!std::isfinite(softmax_scale)) return ISATTN_ERR_UNSUPPORTED;
    const int64_t nq = int64_t(s.batch) * s.seqlen_q * s.heads_q;
    const int64_t nk = int64_t(s.batch) * s.seqlen_k * s.heads_k;
    isattn_status_t st;
    if ((st = check_view(q, nq)) != ISATTN_OK) return st;
    if ((st = check_view(k, nk)) != ISATTN_OK) return st;
    if ((st = check_view(v, nk)) != ISATTN_OK) return st;
    if ((st = check_view(o, nq)) != ISATTN_OK) return st;
    if (nq > 0 && lse == nullptr) return ISATTN_ERR_NULL;
    if (nq > 0) {
        // K/V rows of a head are addressed with 32-bit byte offsets
        const int64_t rk = int64_t(cdiv(s.seqlen_k, kBlock)) * kBlock;
        if (rk * k->stride_s * 2 >= (int64_t(1) << 31) || rk * v->stride_s * 2 >= (int64_t(1) << 31))
            return ISATTN_ERR_STRIDE_ALIGN;
    }
    FwdArgs a{};
    a.mask_kind = ISATTN_MASK_DENSE;
    if (mask != nullptr && mask->kind != ISATTN_MASK_DENSE) {
        if (mask->kind != ISATTN_MASK_BLOCK_CSR) return ISATTN_ERR_MASK;
        if (mask->block_q != kBlock || mask->block_k != kBlock) return ISATTN_ERR_UNSUPPORTED;
        if (mask->heads != 1 && mask->heads != s.heads_k && mask->heads != s.heads_q)
            return ISATTN_ERR_MASK;
        if (mask->q2k_row_ptr == nullptr || mask->q2k_col == nullptr) return ISATTN_ERR_NULL;
        a.mask_kind = ISATTN_MASK_BLOCK_CSR;
        a.Hm = mask->heads;
        a.q2k_ptr = mask->q2k_row_ptr;
        a.q2k_col = mask->q2k_col;
        if (mask->token_bits != nullptr) {
            if ((reinterpret_cast<uintptr_t>(mask->token_bits) & 15u) != 0) return ISATTN_ERR_STRIDE_ALIGN;
            a.tok = mask->token_bits;
        }
    }
    if (varlen != nullptr) {
        if (s.batch > 0 && (varlen->cu_seqlens_q == nullptr || varlen->cu_seqlens_k == nullptr))
            return ISATTN_ERR_NULL;
        a.cu_q = varlen->cu_seqlens_q;
        a.cu_k = varlen->cu_seqlens_k;
    }
    copy_view(q, &a.q, &a.q_sb, &a.q_ss, &a.q_sh);
    copy_view(k, &a.k, &a.k_sb, &a.k_ss, &a.k_sh);
    copy_view(v, &a.v, &a.v_sb, &a.v_ss, &a.v_sh);
    copy_view_out(o, &a.o, &a.o_sb, &a.o_ss, &a.o_sh);
    a.lse = const_cast<float*>(lse);
    a.B = s.batch;
    a.Sq = s.seqlen_q;
    a.Sk = s.seqlen_k;
    a.Hq = s.heads_q;
    a.Hk = s.heads_k;
    a.G = s.heads_q / s.heads_k;
    a.Dqk = s.dim_qk;
    a.Dv = s.dim_v;
    a.n_qb = cdiv(s.seqlen_q, kBlock);
    a.n_kb = cdiv(s.seqlen_k, kBlock);
    a.lse_ld = s.seqlen_q;
    a.causal = causal != 0;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    *args = a;
    return ISATTN_OK;
}

isattn_status_t validate_index(const int32_t* indices, int32_t batch, int32_t seqlen_q,
                               int32_t seqlen_k, int32_t nhk, int32_t topk, int32_t block_q,
                               int32_t block_k, const int32_t* q2k_row_ptr, const int32_t* q2k_col,
                               const int32_t* k2q_row_ptr, const int32_t* k2q_col,
                               int64_t col_capacity, const void* workspace,
                               size_t workspace_bytes, CsrPlan* plan) {
    if (batch < 0 || seqlen_q < 0 || seqlen_k < 0 || nhk < 0 || topk < 0) return ISATTN_ERR_SHAPE;
    if (block_q < 1 || block_k < 1) return ISATTN_ERR_SHAPE;
    const int32_t n_qb = cdiv(seqlen_q, block_q);
    const int32_t n_kb = cdiv(seqlen_k, block_k);
    if (n_kb > kMaxKeyBlocks) return ISATTN_ERR_UNSUPPORTED;
    if (int64_t(batch) * seqlen_q * nhk >= (int64_t(1) << 31)) return ISATTN_ERR_SHAPE;
    const int64_t n_idx = int64_t(batch) * seqlen_q * nhk * topk;
    if (n_idx > 0 && indices == nullptr) return ISATTN_ERR_NULL;
    const int64_t nnz_max = int64_t(batch) * nhk * n_qb * n_kb;
    isattn_status_t st = check_csr_outputs(int64_t(batch) * nhk * n_qb, nnz_max, q2k_row_ptr,
                                           q2k_col, k2q_row_ptr, k2q_col, col_capacity);
    if (st != ISATTN_OK) return st;
    CsrPlan p{};
    if (!plan_csr_workspace(batch, nhk, n_qb, n_kb, true, &p)) return ISATTN_ERR_SHAPE;
    if (workspace_bytes < p.total) return ISATTN_ERR_WORKSPACE;
    if (p.total > 0 && workspace == nullptr) return ISATTN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kWsAlign - 1)) != 0) return ISATTN_ERR_WORKSPACE;
    *plan = p;
    return ISATTN_OK;
}

isattn_status_t validate_blockmask(const uint8_t* presence, int32_t batch, int32_t heads,
                                   int32_t n_qb, int32_t n_kb, const int32_t* q2k_row_ptr,
                                   const int32_t* q2k_col, const int32_t* k2q_row_ptr,
                                   const int32_t* k2q_col, int64_t col_capacity,
                                   const void* workspace, size_t workspace_bytes, CsrPlan* plan) {
    if (batch < 0 || heads < 0 || n_qb < 0 || n_kb < 0) return ISATTN_ERR_SHAPE;
    const int64_t nnz_max = int64_t(batch) * heads * n_qb * n_kb;
    if (nnz_max > 0 && presence == nullptr) return ISATTN_ERR_NULL;
    isattn_status_t st = check_csr_outputs(int64_t(batch) * heads * n_qb, nnz_max, q2k_row_ptr,
                                           q2k_col, k2q_row_ptr, k2q_col, col_capacity);
    if (st != ISATTN_OK) return st;
    CsrPlan p{};
    if (!plan_csr_workspace(batch, heads, n_qb, n_kb, false, &p)) return ISATTN_ERR_SHAPE;
    if (workspace_bytes < p.total) return ISATTN_ERR_WORKSPACE;
    if (p.total > 0 && workspace == nullptr) return ISATTN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kWsAlign - 1)) != 0) return ISATTN_ERR_WORKSPACE;
    *plan = p;
    return ISATTN_OK;
}

}  // namespace isattn
